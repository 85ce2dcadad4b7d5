// host_check.cpp -- CPU checks of the library's host-only code
// (vla_flow_matching_amd/csrc/host_pack.h): configuration checks over a
// fuzzed set of configurations, blob sizes, and the weight repacks, whose
// results are checked against properties that follow from the blob layout
// and the packed layouts' definitions (every source row used exactly once,
// rotary partners and gate/up partners 16 rows apart, the norm scales, the
// fold of action_in_proj computed naively in double).  Built and run under
// AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_sanitizers.py; exits 0 when every check holds.
#include <climits>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <map>
#include <random>
#include <vector>

#include "host_pack.h"

using namespace pi0x::hostpack;

static int g_fail = 0;
#define CHECK(cond, ...)                      \
  do {                                        \
    if (!(cond)) {                            \
      ++g_fail;                               \
      if (g_fail <= 20) {                     \
        std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
        std::fprintf(stderr, __VA_ARGS__);    \
        std::fprintf(stderr, "\n");           \
      }                                       \
    }                                         \
  } while (0)

static pi0x_config default_config() {
  pi0x_config c{};
  c.width = 1024; c.depth = 18; c.mlp_dim = 4096; c.num_heads = 8; c.num_kv_heads = 1; c.head_dim = 256;
  c.action_horizon = 50; c.action_dim = 32; c.state_dim = 32; c.max_batch = 64; c.max_prefix_len = 1024;
  c.max_steps = 64; c.rms_eps = 1e-6f; c.rope_theta = 10000.f; c.time_min_period = 4e-3f; c.time_max_period = 4.f;
  c.dtype = PI0X_BF16; c.use_graphs = 1;
  return c;
}

static void check_configs() {
  std::string msg;
  pi0x_config c = default_config();
  CHECK(config_error(&c, &msg) == PI0X_OK, "default config rejected: %s", msg.c_str());
  CHECK(prefix_config_error(&c, 1 << 16, &msg) == PI0X_OK, "default prefix config rejected: %s", msg.c_str());
  CHECK(config_error(nullptr, &msg) == PI0X_ERR_INVALID_ARG, "NULL config");
  // the pi0 expert's blob: 18 layers of 1024-wide Gemma plus the action head
  const size_t layer = 1024 + 2048 * 1024 + 2 * 256 * 1024 + 1024 * 2048 + 1024 + 3 * 4096 * 1024;
  CHECK(weight_count(&c) == layer * 18 + 1024 + (1024 * 32 + 1024) * 2 + (1024 * 2048 + 1024) + (1024 * 1024 + 1024) +
                                (32 * 1024 + 32),
        "pi0 weight count");
  CHECK(prefix_weight_count(&c) == layer * 18, "prefix weight count");
  struct Bad {
    void (*edit)(pi0x_config&);
    pi0x_status want;
  };
  const Bad bad[] = {
      {[](pi0x_config& k) { k.width = 0; }, PI0X_ERR_INVALID_ARG},
      {[](pi0x_config& k) { k.depth = -3; }, PI0X_ERR_INVALID_ARG},
      {[](pi0x_config& k) { k.max_prefix_len = -1; }, PI0X_ERR_INVALID_ARG},
      {[](pi0x_config& k) { k.dtype = (pi0x_dtype)7; }, PI0X_ERR_DTYPE},
      {[](pi0x_config& k) { k.rms_eps = NAN; }, PI0X_ERR_INVALID_ARG},
      {[](pi0x_config& k) { k.rope_theta = 0.f; }, PI0X_ERR_INVALID_ARG},
      {[](pi0x_config& k) { k.num_kv_heads = 2; }, PI0X_ERR_SHAPE},
      {[](pi0x_config& k) { k.head_dim = 96; }, PI0X_ERR_SHAPE},
      {[](pi0x_config& k) { k.width = 1000; }, PI0X_ERR_SHAPE},
      {[](pi0x_config& k) { k.mlp_dim = 4000; }, PI0X_ERR_SHAPE},
      {[](pi0x_config& k) { k.num_heads = 3; k.head_dim = 32; }, PI0X_ERR_SHAPE},
      {[](pi0x_config& k) { k.action_dim = 65; }, PI0X_ERR_SHAPE},
      {[](pi0x_config& k) { k.num_heads = INT_MAX; }, PI0X_ERR_CAPACITY},
      {[](pi0x_config& k) { k.max_batch = INT_MAX; }, PI0X_ERR_CAPACITY},
      {[](pi0x_config& k) { k.width = 1 << 30; }, PI0X_ERR_CAPACITY},
  };
  for (const Bad& b : bad) {
    pi0x_config k = default_config();
    b.edit(k);
    const pi0x_status st = config_error(&k, &msg);
    CHECK(st == b.want, "bad config: status %d, expected %d (%s)", (int)st, (int)b.want, msg.c_str());
  }
  // fuzz: every field drawn from values around the limits; the checks must
  // never overflow (UBSan) and whatever they accept must size sanely
  std::mt19937_64 rng(12345);
  const int vals[] = {INT_MIN, -1, 0, 1, 2, 7, 16, 31, 32, 64, 65, 128, 256, 1000, 1024, 2048, 4096,
                      1 << 16, (1 << 16) + 256, 1 << 20, 1 << 24, INT_MAX - 255, INT_MAX};
  auto pick = [&]() { return vals[rng() % (sizeof(vals) / sizeof(vals[0]))]; };
  int accepted = 0;
  for (int it = 0; it < 200000; ++it) {
    pi0x_config k = default_config();
    int* fields[] = {&k.width, &k.depth, &k.mlp_dim, &k.num_heads, &k.num_kv_heads, &k.head_dim,
                     &k.action_horizon, &k.action_dim, &k.state_dim, &k.max_batch, &k.max_prefix_len, &k.max_steps};
    const int nf = 1 + (int)(rng() % 4);
    for (int f = 0; f < nf; ++f) *fields[rng() % 12] = pick();
    if (config_error(&k, &msg) == PI0X_OK) {
      ++accepted;
      CHECK(weight_count(&k) > prefix_weight_count(&k), "accepted config with a non-growing blob");
      CHECK(k.width <= (1 << 16) && (long long)k.max_batch * (k.action_horizon + 1) <= (1LL << 24),
            "accepted config beyond the limits");
    }
    (void)prefix_config_error(&k, 1 << 16, &msg);
  }
  CHECK(accepted > 0, "the fuzz accepted nothing");
}

// bf16 rounding: exact values stay, ties go to even, NaN and infinity survive
static void check_bf16() {
  auto bits = [](float f) {
    uint32_t u;
    std::memcpy(&u, &f, 4);
    return u;
  };
  auto from = [](uint32_t u) {
    float f;
    std::memcpy(&f, &u, 4);
    return f;
  };
  CHECK(to_bf16(1.0f) == 0x3f80, "1.0");
  CHECK(to_bf16(-2.5f) == 0xc020, "-2.5");
  CHECK(to_bf16(from(0x3f808000u)) == 0x3f80, "tie to even (down)");
  CHECK(to_bf16(from(0x3f818000u)) == 0x3f82, "tie to even (up)");
  CHECK(to_bf16(from(0x3f808001u)) == 0x3f81, "above the tie");
  CHECK(to_bf16(INFINITY) == 0x7f80, "inf");
  const uint16_t n = to_bf16(NAN);
  CHECK((n & 0x7f80) == 0x7f80 && (n & 0x7f) != 0, "NaN");
  CHECK(to_bf16(from(0x7f800001u)) != 0x7f80, "signalling NaN must not become inf");
  CHECK(bits(round_model(1.00390625f, true)) == 0x3f800000u, "round_model ties to 1.0");
  CHECK(round_model(1.00390625f, false) == 1.00390625f, "fp32 passes through");
}

// A blob of random values that bf16 holds exactly (8 significant bits,
// exponents within +-8), so packing never rounds them; a packed row is traced
// back to its source by matching the whole row.
struct Blob {
  std::vector<float> v;
  std::map<float, std::vector<size_t>> where;  // value -> its indices
};

static Blob make_blob(size_t n, bool zero_norms, const Dims& d, int depth) {
  Blob b;
  b.v.resize(n);
  std::mt19937_64 rng(7);
  for (size_t k = 0; k < n; ++k) {
    const uint64_t r = rng();
    const float m = (float)(128 + (r & 127));
    const int e = (int)((r >> 7) % 17) - 8 - 7;
    b.v[k] = std::ldexp(m, e) * (((r >> 12) & 1) ? -1.f : 1.f);
  }
  // zeroed norm weights: (1 + w) = 1, so packed values equal their sources
  if (zero_norms) {
    for (int l = 0; l < depth; ++l) {
      const LayerSrc s = layer_src(b.v.data(), d, l);
      std::fill(const_cast<float*>(s.in_norm), const_cast<float*>(s.in_norm) + d.W, 0.f);
      std::fill(const_cast<float*>(s.post), const_cast<float*>(s.post) + d.W, 0.f);
    }
    const HeadSrc h = head_src(b.v.data(), d, depth);
    std::fill(const_cast<float*>(h.final_norm), const_cast<float*>(h.final_norm) + d.W, 0.f);
  }
  for (size_t i = 0; i < n; ++i) b.where[b.v[i]].push_back(i);
  return b;
}

template <typename E>
static float elem_value(E e);
template <>
float elem_value<float>(float e) { return e; }
template <>
float elem_value<uint16_t>(uint16_t e) {
  const uint32_t u = (uint32_t)e << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// index in the blob where packed row r's W values start as one contiguous
// run; SIZE_MAX if there is none (or the row matches in more than one place)
template <typename E>
static size_t source_row(const Blob& b, const std::vector<E>& p, size_t r, int W) {
  auto it = b.where.find(elem_value<E>(p[r * W]));
  if (it == b.where.end()) return SIZE_MAX;
  size_t found = SIZE_MAX;
  for (size_t start : it->second) {
    if (start + W > b.v.size()) continue;
    bool same = true;
    for (int k = 1; k < W && same; ++k) same = elem_value<E>(p[r * W + k]) == b.v[start + k];
    if (same) {
      if (found != SIZE_MAX) return SIZE_MAX;
      found = start;
    }
  }
  return found;
}

template <typename E>
static void check_packs(const Dims& d, int depth) {
  pi0x_config c = default_config();
  c.width = d.W; c.mlp_dim = d.M; c.num_heads = d.nh; c.head_dim = d.dh; c.depth = depth;
  c.action_dim = d.A; c.state_dim = d.Sd;
  const size_t n = weight_count(&c);
  const Blob b = make_blob(n, true, d, depth);
  const int W = d.W, dh = d.dh, qd = d.qd(), M = d.M;
  for (int l = 0; l < depth; ++l) {
    const LayerSrc s = layer_src(b.v.data(), d, l);
    const size_t q0 = s.wq - b.v.data(), k0 = s.wk - b.v.data(), v0 = s.wv - b.v.data();
    // q/k/v: a bijection onto the q, k and v rows; rotary partners 16 apart
    const std::vector<E> qkv = pack_qkv<E>(s, d);
    CHECK(qkv.size() == (size_t)(qd + 2 * dh) * W, "qkv size");
    std::vector<int> used(qd + 2 * dh, 0);
    for (int r = 0; r < qd + 2 * dh; ++r) {
      const size_t src = source_row(b, qkv, r, W);
      CHECK(src != SIZE_MAX && (src - q0) % W == 0, "qkv row %d is not a whole source row", r);
      if (src == SIZE_MAX) continue;
      const size_t orow = (src - q0) / W;  // row in [q; k; v]
      CHECK(orow < (size_t)(qd + 2 * dh), "qkv row %d out of range", r);
      if (orow < (size_t)(qd + 2 * dh)) ++used[orow];
      if (r < qd + dh) {
        CHECK((r < qd) == (src < k0), "qkv row %d: query/key block", r);
        if (r % 32 < 16) {  // partner: packed row r + 16 holds original row + dh/2
          const size_t src2 = source_row(b, qkv, r + 16, W);
          CHECK(src2 != SIZE_MAX && src2 == src + (size_t)(dh / 2) * W, "qkv rows %d/%d are not rotary partners", r,
                r + 16);
        }
      } else {
        CHECK(src >= v0 && src == v0 + (size_t)(r - qd - dh) * W, "value row %d", r);
      }
    }
    for (int r = 0; r < qd + 2 * dh; ++r) CHECK(used[r] == 1, "source q/k/v row %d used %d times", r, used[r]);
    // gate/up: gate row j and up row j sit 16 apart in each 32-row group
    const std::vector<E> gu = pack_gate_up<E>(s, d);
    const size_t g0 = s.wg - b.v.data(), u0 = s.wu - b.v.data();
    for (int r = 0; r < 2 * M; ++r) {
      const size_t src = source_row(b, gu, r, W);
      const int j = (r / 32) * 16 + r % 16;
      const size_t want = (r % 32 < 16 ? g0 : u0) + (size_t)j * W;
      CHECK(src == want, "gate/up row %d", r);
    }
    // o and down as is
    const std::vector<E> o = pack_plain<E>(s.wo, (size_t)W * qd), dn = pack_plain<E>(s.wd, (size_t)W * M);
    for (size_t i = 0; i < o.size(); i += 97) CHECK(elem_value<E>(o[i]) == s.wo[i], "o_proj element %zu", i);
    for (size_t i = 0; i < dn.size(); i += 97) CHECK(elem_value<E>(dn[i]) == s.wd[i], "down element %zu", i);
  }
  // the norm scales: with norm weights w the packed columns are source * (1 + w)
  {
    Blob b2 = make_blob(n, true, d, depth);
    LayerSrc s = layer_src(b2.v.data(), d, 0);
    for (int k = 0; k < W; ++k) {
      const_cast<float*>(s.in_norm)[k] = (float)(k % 7) * 0.25f;
      const_cast<float*>(s.post)[k] = -(float)(k % 5) * 0.125f;
    }
    const std::vector<E> qkv = pack_qkv<E>(s, d), gu = pack_gate_up<E>(s, d);
    const std::vector<E> qkv1 = pack_qkv<E>(layer_src(b.v.data(), d, 0), d);
    const std::vector<E> gu1 = pack_gate_up<E>(layer_src(b.v.data(), d, 0), d);
    for (int r = 0; r < qd + 2 * dh; r += 3)
      for (int k = 0; k < W; ++k) {
        const float want = elem_value<E>(to_elem<E>(elem_value<E>(qkv1[(size_t)r * W + k]) * (1.f + (float)(k % 7) * 0.25f)));
        CHECK(elem_value<E>(qkv[(size_t)r * W + k]) == want, "qkv scale r %d k %d", r, k);
      }
    for (int r = 0; r < 2 * M; r += 5)
      for (int k = 0; k < W; ++k) {
        const float want = elem_value<E>(to_elem<E>(elem_value<E>(gu1[(size_t)r * W + k]) * (1.f - (float)(k % 5) * 0.125f)));
        CHECK(elem_value<E>(gu[(size_t)r * W + k]) == want, "gate/up scale r %d k %d", r, k);
      }
  }
  // the head
  const HeadSrc h = head_src(b.v.data(), d, depth);
  CHECK(h.bout + d.A == b.v.data() + n, "head layout ends at the blob's end");
  const std::vector<E> tt = pack_time_half<E>(h, d);
  for (int r = 0; r < W; ++r) {
    const size_t src = source_row(b, tt, r, W);
    CHECK(src == (size_t)(h.wmi - b.v.data()) + (size_t)r * 2 * W + W, "time half row %d", r);
  }
  const int Apad = 128;
  const std::vector<E> op = pack_out_proj<E>(h, d, Apad);
  CHECK(op.size() == (size_t)Apad * W, "out proj size");
  for (int r = 0; r < Apad; ++r) {
    if (r < d.A) {
      CHECK(source_row(b, op, r, W) == (size_t)(h.wout - b.v.data()) + (size_t)r * W, "out proj row %d", r);
    } else {
      for (int k = 0; k < W; ++k) CHECK(elem_value<E>(op[(size_t)r * W + k]) == 0.f, "out proj padding row %d", r);
    }
  }
  std::vector<float> comb, bias;
  fold_action_in(h, d, &comb, &bias);
  CHECK(comb.size() == (size_t)W * d.A && bias.size() == (size_t)W, "fold sizes");
  for (int o = 0; o < W; o += 7) {
    double bsum = round_model(h.bmi[o], d.bf16);
    for (int k = 0; k < W; ++k) bsum += (double)round_model(h.wmi[(size_t)o * 2 * W + k], d.bf16) * round_model(h.bi[k], d.bf16);
    CHECK(std::fabs(bias[o] - bsum) <= 1e-6 * (1 + std::fabs(bsum)), "fold bias %d", o);
    for (int a = 0; a < d.A; ++a) {
      double sum = 0;
      for (int k = 0; k < W; ++k)
        sum += (double)round_model(h.wmi[(size_t)o * 2 * W + k], d.bf16) * round_model(h.wi[(size_t)k * d.A + a], d.bf16);
      CHECK(std::fabs(comb[(size_t)a * W + o] - sum) <= 1e-6 * (1 + std::fabs(sum)), "fold %d %d", o, a);
    }
  }
  const std::vector<float> sm = pack_small(h.ws, (size_t)W * d.Sd, d.bf16);
  for (size_t i = 0; i < sm.size(); i += 13) CHECK(sm[i] == h.ws[i], "state_proj element %zu", i);
}

int main() {
  check_configs();
  check_bf16();
  // two small shapes: head_dim 32 (one 32-row group per head) and 64
  check_packs<float>(Dims{256, 256, 4, 32, 8, 8, false}, 2);
  check_packs<uint16_t>(Dims{256, 256, 4, 32, 8, 8, true}, 2);
  check_packs<float>(Dims{256, 384, 2, 64, 5, 3, false}, 1);
  check_packs<uint16_t>(Dims{256, 384, 2, 64, 5, 3, true}, 1);
  if (g_fail) {
    std::fprintf(stderr, "%d check(s) failed\n", g_fail);
    return 1;
  }
  std::printf("host checks passed\n");
  return 0;
}
