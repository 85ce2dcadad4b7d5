/*
 * sanitize_driver.c -- runs the fp64 oracle (pi0_oracle.c) from a case file,
 * so that a build under AddressSanitizer and UndefinedBehaviorSanitizer can
 * exercise it as a plain executable (no sanitizer runtime has to be preloaded
 * into Python).
 *
 * TEST INFRASTRUCTURE ONLY, like the oracle: built and run by
 * tests/test_sanitizers.py, which writes the case files and compares the
 * outputs with the ordinary build of the oracle.
 *
 * Case file (little endian), read field by field:
 *   char[8]  "PI0OSAN1"
 *   int32    mode: 0 denoise_ex, 1 velocity, 2 prefill
 *   int32[9] width depth mlp_dim num_heads num_kv_heads head_dim horizon action_dim state_dim
 *   double[4] rms_eps rope_theta min_period max_period
 *   int32[7] L valid num_steps schedule x_prediction causal has_blend
 *   double[2] pos_shift t
 *   then float64 arrays:
 *     mode 0: weights, state[state_dim], noise[H*A], kv[depth*2*L*kd],
 *             and with has_blend dof_mask[H*A], padding[H*A]
 *     mode 1: weights, state, x[H*A], kv
 *     mode 2: layer weights, embeddings[L*width]
 * Output file: the result as float64 (mode 0/1: [H*A]; mode 2: the cache
 * [depth][2][L][kd]).
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int width, depth, mlp_dim, num_heads, num_kv_heads, head_dim;
  int horizon, action_dim, state_dim;
  double rms_eps, rope_theta, min_period, max_period;
} pi0o_cfg;

size_t pi0o_weight_count(const pi0o_cfg* c);
size_t pi0o_prefill_weight_count(const pi0o_cfg* c);
void pi0o_velocity(const pi0o_cfg* c, const double* w, const double* state, const double* x, double t,
                   const double* kv, int L, int valid, double pos_shift, int causal, double* v);
void pi0o_denoise_ex(const pi0o_cfg* c, const double* w, const double* state, const double* noise,
                     const double* kv, int L, int valid, int num_steps, double pos_shift, int schedule,
                     int x_pred, int causal, const double* dof_mask, const double* padding, double* out);
void pi0o_prefill(const pi0o_cfg* c, const double* w, const double* emb, int L, int valid, double pos_shift,
                  double* kv_out);

static FILE* g_in;

static void die(const char* m) {
  fprintf(stderr, "sanitize_driver: %s\n", m);
  exit(2);
}

static void get(void* p, size_t bytes) {
  if (bytes && fread(p, 1, bytes, g_in) != bytes) die("short case file");
}

/* n doubles from the case file, in a buffer of exactly that size (a zero
 * count still gets a valid, empty allocation) */
static double* get_array(size_t n) {
  double* a = (double*)malloc(n ? n * sizeof(double) : 1);
  if (!a) die("out of memory");
  get(a, n * sizeof(double));
  return a;
}

int main(int argc, char** argv) {
  if (argc != 3) die("usage: sanitize_driver CASE OUT");
  g_in = fopen(argv[1], "rb");
  if (!g_in) die("cannot open the case file");
  char magic[8];
  get(magic, 8);
  if (memcmp(magic, "PI0OSAN1", 8) != 0) die("bad magic");
  int32_t mode, ci[9], p[7];
  double cd[4], pd[2];
  get(&mode, 4);
  get(ci, sizeof ci);
  get(cd, sizeof cd);
  get(p, sizeof p);
  get(pd, sizeof pd);
  pi0o_cfg c = {ci[0], ci[1], ci[2], ci[3], ci[4], ci[5], ci[6], ci[7], ci[8], cd[0], cd[1], cd[2], cd[3]};
  const int L = p[0], valid = p[1], steps = p[2], schedule = p[3], xpred = p[4], causal = p[5], blend = p[6];
  const size_t HA = (size_t)c.horizon * c.action_dim, kd = (size_t)c.num_kv_heads * c.head_dim;
  const size_t nkv = (size_t)c.depth * 2 * (size_t)L * kd;
  double* out = NULL;
  size_t nout = 0;
  if (mode == 0 || mode == 1) {
    double* w = get_array(pi0o_weight_count(&c));
    double* state = get_array((size_t)c.state_dim);
    double* x = get_array(HA);
    double* kv = get_array(nkv);
    double *mask = NULL, *pad = NULL;
    if (mode == 0 && blend) {
      mask = get_array(HA);
      pad = get_array(HA);
    }
    nout = HA;
    out = (double*)malloc(nout * sizeof(double));
    if (!out) die("out of memory");
    if (mode == 0)
      pi0o_denoise_ex(&c, w, state, x, kv, L, valid, steps, pd[0], schedule, xpred, causal, mask, pad, out);
    else
      pi0o_velocity(&c, w, state, x, pd[1], kv, L, valid, pd[0], causal, out);
    free(w);
    free(state);
    free(x);
    free(kv);
    free(mask);
    free(pad);
  } else if (mode == 2) {
    double* w = get_array(pi0o_prefill_weight_count(&c));
    double* emb = get_array((size_t)L * c.width);
    nout = nkv;
    out = (double*)malloc(nout ? nout * sizeof(double) : 1);
    if (!out) die("out of memory");
    pi0o_prefill(&c, w, emb, L, valid, pd[0], out);
    free(w);
    free(emb);
  } else {
    die("unknown mode");
  }
  fclose(g_in);
  FILE* f = fopen(argv[2], "wb");
  if (!f) die("cannot open the output file");
  if (nout && fwrite(out, sizeof(double), nout, f) != nout) die("short write");
  fclose(f);
  free(out);
  return 0;
}
