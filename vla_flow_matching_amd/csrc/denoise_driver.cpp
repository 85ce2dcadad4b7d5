// denoise_driver: the denoise loop through the C ABI from a plain C++ process.
//
// Builds a bf16 expert of the pi0 shape (pi0x_config_default) with seeded
// uniform weights (standard deviation 0.02), puts the inputs in device memory
// (prefix K/V, valid lengths = prefix_len, state and noise), and makes
// `--calls` pi0x_denoise calls, each synchronized.  With
// --eager the calls run their kernels directly (no captured graph), as the
// library's kernel-timing mode does.  With
// --copy-calibration-mib M it first copies M MiB device to device once, a
// transfer of known size against which hardware byte counters are scaled.
// It is what hardware-counter runs (rocprofv3 --pmc) execute: no Python, no
// torch, one process that only does this.
//
//   denoise_driver [--batch B] [--prefix-len L] [--steps N] [--calls C] [--eager] [--copy-calibration-mib M]
//
// Exit status 0 on success; any failing call prints pi0x_last_error() and exits 1.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "pi0x.h"

namespace {

void hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    std::fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    std::exit(1);
  }
}

void pi0x_check(pi0x_status s, const char* what) {
  if (s != PI0X_OK) {
    std::fprintf(stderr, "%s: status %d: %s\n", what, (int)s, pi0x_last_error());
    std::exit(1);
  }
}

// splitmix64: a seeded stream of uniform doubles in [0, 1)
struct Rng {
  uint64_t s;
  double next() {
    uint64_t z = (s += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    z ^= z >> 31;
    return (double)(z >> 11) * (1.0 / 9007199254740992.0);
  }
  // uniform with the given standard deviation, centred on 0
  float uniform_sd(double sd) { return (float)((next() * 2.0 - 1.0) * sd * 1.7320508075688772); }
};

uint16_t to_bf16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

int arg_int(int argc, char** argv, const char* name, int def) {
  for (int i = 1; i + 1 < argc; ++i)
    if (std::strcmp(argv[i], name) == 0) return std::atoi(argv[i + 1]);
  return def;
}

bool arg_flag(int argc, char** argv, const char* name) {
  for (int i = 1; i < argc; ++i)
    if (std::strcmp(argv[i], name) == 0) return true;
  return false;
}

}  // namespace

int main(int argc, char** argv) {
  const int B = arg_int(argc, argv, "--batch", 64);
  const int L = arg_int(argc, argv, "--prefix-len", 816);
  const int N = arg_int(argc, argv, "--steps", 10);
  const int calls = arg_int(argc, argv, "--calls", 1);
  const int calib_mib = arg_int(argc, argv, "--copy-calibration-mib", 0);
  if (B < 1 || L < 0 || N < 1 || calls < 0 || calib_mib < 0) {
    std::fprintf(stderr, "bad arguments\n");
    return 1;
  }

  pi0x_config cfg;
  pi0x_config_default(&cfg);
  cfg.max_batch = B;
  cfg.max_prefix_len = L > 0 ? L : 1;
  if (cfg.max_steps < N) cfg.max_steps = N;
  if (arg_flag(argc, argv, "--eager")) cfg.use_graphs = 0;
  const size_t nw = pi0x_weight_count(&cfg);
  if (nw == 0) {
    std::fprintf(stderr, "pi0x_weight_count: invalid config\n");
    return 1;
  }
  Rng rng{12345};
  std::vector<float> w(nw);
  for (float& x : w) x = rng.uniform_sd(0.02);
  pi0x_expert* h = nullptr;
  pi0x_check(pi0x_expert_create(&cfg, w.data(), nw * sizeof(float), &h), "pi0x_expert_create");
  w.clear();
  w.shrink_to_fit();

  const int D = cfg.depth, dh = cfg.head_dim, H = cfg.action_horizon, A = cfg.action_dim, Sd = cfg.state_dim;
  const size_t n_kv = (size_t)D * 2 * B * L * dh;
  std::vector<uint16_t> kv_h(n_kv);
  for (uint16_t& x : kv_h) x = to_bf16(rng.uniform_sd(1.0));
  std::vector<int32_t> valid_h(B, L);
  std::vector<float> state_h((size_t)B * Sd), noise_h((size_t)B * H * A);
  for (float& x : state_h) x = rng.uniform_sd(1.0);
  for (float& x : noise_h) x = rng.uniform_sd(1.0);

  void *kv = nullptr, *valid = nullptr, *state = nullptr, *noise = nullptr, *out = nullptr;
  hip_check(hipMalloc(&kv, n_kv * 2 + 16), "hipMalloc kv");
  hip_check(hipMalloc(&valid, B * sizeof(int32_t)), "hipMalloc valid");
  hip_check(hipMalloc(&state, state_h.size() * 4), "hipMalloc state");
  hip_check(hipMalloc(&noise, noise_h.size() * 4), "hipMalloc noise");
  hip_check(hipMalloc(&out, noise_h.size() * 4), "hipMalloc out");
  hip_check(hipMemcpy(kv, kv_h.data(), n_kv * 2, hipMemcpyHostToDevice), "copy kv");
  hip_check(hipMemcpy(valid, valid_h.data(), B * sizeof(int32_t), hipMemcpyHostToDevice), "copy valid");
  hip_check(hipMemcpy(state, state_h.data(), state_h.size() * 4, hipMemcpyHostToDevice), "copy state");
  hip_check(hipMemcpy(noise, noise_h.data(), noise_h.size() * 4, hipMemcpyHostToDevice), "copy noise");
  kv_h.clear();
  kv_h.shrink_to_fit();

  if (calib_mib > 0) {
    const size_t bytes = (size_t)calib_mib << 20;
    void *a = nullptr, *b = nullptr;
    hip_check(hipMalloc(&a, bytes), "hipMalloc calibration");
    hip_check(hipMalloc(&b, bytes), "hipMalloc calibration");
    hip_check(hipMemset(a, 0, bytes), "hipMemset calibration");
    hip_check(hipMemcpy(b, a, bytes, hipMemcpyDeviceToDevice), "calibration copy");
    hip_check(hipDeviceSynchronize(), "calibration sync");
    hip_check(hipFree(a), "hipFree");
    hip_check(hipFree(b), "hipFree");
  }

  for (int c = 0; c < calls; ++c) {
    pi0x_check(pi0x_denoise(h, B, L, kv, (const int32_t*)valid, (const float*)state, (const float*)noise, N,
                            (float*)out, nullptr),
               "pi0x_denoise");
    hip_check(hipDeviceSynchronize(), "denoise sync");
  }
  std::vector<float> out_h(noise_h.size());
  hip_check(hipMemcpy(out_h.data(), out, out_h.size() * 4, hipMemcpyDeviceToHost), "copy out");
  double s = 0.0;
  for (float x : out_h) s += (double)x * x;
  std::printf("denoise_driver: batch %d prefix_len %d steps %d calls %d, output mean square %.6g\n", B, L, N, calls,
              s / (double)out_h.size());

  pi0x_expert_destroy(h);
  hip_check(hipFree(kv), "hipFree");
  hip_check(hipFree(valid), "hipFree");
  hip_check(hipFree(state), "hipFree");
  hip_check(hipFree(noise), "hipFree");
  hip_check(hipFree(out), "hipFree");
  return 0;
}
