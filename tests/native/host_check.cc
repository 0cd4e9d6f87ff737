// The library's host-side logic (onebit_host.hpp: argument and
// hyper-parameter checks, the overlap check, byte counts, the workspace
// layout, the tensor table) on the CPU, fuzzed against brute-force
// references.  Built with AddressSanitizer and UndefinedBehaviorSanitizer
// by tests/test_host_sanitized.py: any out-of-bounds access, leak, signed
// overflow or other undefined behaviour aborts it, and every disagreement
// with a reference is counted and printed.
#include <algorithm>
#include <cinttypes>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <limits>
#include <random>
#include <vector>

#include "onebit_host.hpp"

using namespace onebit_host;
typedef __int128 i128;

static int g_fail = 0;

#define EXPECT(cond, ...)                                   \
  do {                                                      \
    if (!(cond)) {                                          \
      if (g_fail < 40) {                                    \
        std::printf("FAIL %s:%d: ", __FILE__, __LINE__);    \
        std::printf(__VA_ARGS__);                           \
        std::printf("\n");                                  \
      }                                                     \
      ++g_fail;                                             \
    }                                                       \
  } while (0)

static const int32_t kChunks[] = {64,   128,   256,   512,     1024,    2048,
                                   4096, 8192,  16384, 32768, 65536, 1 << 20, 1 << 24};
static const int kNChunks = sizeof kChunks / sizeof kChunks[0];

// Reference for the size bounds, written out per chunk size: the threads of
// one chunk's workgroup with four float4 slots per thread (the entry points
// that take n and chunk; one 64-wide wave up to 1024 elements), and the
// widest a table kernel launches (the warmup passes' two slots at 4096);
// chunks longer than 16384 take 256 threads that walk the chunk in blocks.
// A launch of k chunks fits when k <= 2^30 - 1 and k * threads < 2^32.
static int64_t ref_threads(int32_t chunk, bool table) {
  switch (chunk) {
    case 64: case 128: case 256: case 512: case 1024: return 64;
    case 2048: return 128;
    case 4096: return table ? 512 : 256;
    case 8192: return 512;
    case 16384: return 1024;
    default: return 256;
  }
}
static bool ref_fits(i128 k, int32_t chunk, bool table) {
  return k <= (i128)(1 << 30) - 1 && k * ref_threads(chunk, table) <= (i128)0xFFFFFFFFu;
}
// The largest n whose chunks fit.
static int64_t ref_max_n(int32_t chunk, bool table) {
  i128 k = (i128)(1 << 30) - 1;
  while (!ref_fits(k, chunk, table)) k = (i128)0xFFFFFFFFu / ref_threads(chunk, table);
  return (int64_t)(k * chunk);
}

// ---------------------------------------------------------------------------
// tables
// ---------------------------------------------------------------------------
// Reference: the tensor of element i by binary search on the offsets, and
// the (chunk, tensor) segments listed pair by pair in their numbering order.
static void check_table(const std::vector<int64_t>& numels, int32_t chunk, bool per_element) {
  const int32_t L = (int32_t)numels.size();
  HostTable t;
  const int rc = build_table(numels.data(), L, chunk, t, "fuzz");
  EXPECT(rc == ONEBIT_OK, "build_table rc %d (%s)", rc, last_error_slot().c_str());
  if (rc) return;
  std::vector<int64_t> off(L + 1, 0);
  for (int32_t l = 0; l < L; ++l) off[l + 1] = off[l] + numels[l];
  const int64_t N = off[L];
  const int64_t K = (N + chunk - 1) / chunk;
  EXPECT(t.N == N && t.K == K && t.L == L && t.chunk == chunk, "sizes N %lld K %lld", (long long)t.N,
         (long long)t.K);
  EXPECT(t.off == off, "offsets differ");
  auto tensor_of = [&](int64_t i) {
    return (int32_t)(std::upper_bound(off.begin(), off.end(), i) - off.begin() - 1);
  };
  if (per_element) {
    // every element's tensor lies within its chunk's [l0, l1]
    for (int64_t i = 0; i < N; ++i) {
      const int64_t k = i / chunk;
      const int32_t l = tensor_of(i);
      if (!(t.l0[k] <= l && l <= t.l1[k])) {
        EXPECT(false, "element %lld of tensor %d outside chunk %lld's [%d, %d]", (long long)i, l,
               (long long)k, t.l0[k], t.l1[k]);
        break;
      }
    }
  }
  // segments in numbering order
  std::vector<std::vector<int64_t>> by_tensor(L);
  int64_t s = 0;
  for (int64_t k = 0; k < K; ++k) {
    const int64_t first = k * chunk;
    const int64_t last = std::min((k + 1) * (int64_t)chunk, N) - 1;
    const int32_t a = tensor_of(first), b = tensor_of(last);
    EXPECT(t.l0[k] == a && t.l1[k] == b, "chunk %lld: [%d, %d] against [%d, %d]", (long long)k,
           t.l0[k], t.l1[k], a, b);
    EXPECT(t.seg[k] == s, "chunk %lld: seg %d against %lld", (long long)k, t.seg[k], (long long)s);
    for (int32_t l = a; l <= b; ++l) by_tensor[l].push_back(s++);
  }
  EXPECT(t.S == s, "S %lld against %lld", (long long)t.S, (long long)s);
  EXPECT((int64_t)t.lseg[L] == s, "lseg[L] %d", t.lseg[L]);
  // a tensor's segments are the contiguous range [lseg[l], lseg[l+1])
  for (int32_t l = 0; l < L; ++l) {
    const std::vector<int64_t>& v = by_tensor[l];
    bool okl = !v.empty() && t.lseg[l] == v.front() && t.lseg[l + 1] == v.back() + 1 &&
               (int64_t)v.size() == v.back() - v.front() + 1;
    EXPECT(okl, "tensor %d: segments [%d, %d) do not match", l, t.lseg[l], t.lseg[l + 1]);
    if (!okl) break;
  }
}

static std::vector<int64_t> random_numels(std::mt19937_64& r, int32_t chunk) {
  std::uniform_int_distribution<int> nl(1, 400);
  const int L = nl(r);
  std::vector<int64_t> v;
  for (int l = 0; l < L; ++l) {
    const double u = std::uniform_real_distribution<double>(0, 1)(r);
    int64_t n;
    if (u < 0.15) n = chunk * std::uniform_int_distribution<int64_t>(1, 4)(r);   // whole chunks
    else if (u < 0.35) n = std::uniform_int_distribution<int64_t>(1, 9)(r);      // tiny
    else if (u < 0.45) n = chunk - std::uniform_int_distribution<int64_t>(0, 2)(r) + 1;
    else n = (int64_t)std::exp(std::uniform_real_distribution<double>(0, std::log(5.0 * chunk))(r)) + 1;
    v.push_back(n);
  }
  return v;
}

static void fuzz_tables() {
  std::mt19937_64 r(1);
  for (int it = 0; it < 400; ++it) {
    const int32_t chunk = kChunks[it % kNChunks];
    check_table(random_numels(r, chunk), chunk, it % 4 == 0 && chunk <= 65536);
  }
  // edge shapes: one element, exactly one chunk, one chunk plus one, many
  // one-element tensors in one chunk, a tensor ending on every boundary
  for (int32_t chunk : kChunks) {
    if (chunk > 65536) {
      check_table({1}, chunk, true);
      check_table({chunk, 1, chunk - 1, 3}, chunk, false);
      continue;
    }
    check_table({1}, chunk, true);
    check_table({chunk}, chunk, true);
    check_table({chunk + 1}, chunk, true);
    check_table(std::vector<int64_t>(3 * chunk + 5, 1), chunk, false);
    check_table({chunk, chunk, 1, chunk - 1, 2 * chunk}, chunk, true);
    check_table({(int64_t)chunk * 1000 + 7, 3, (int64_t)chunk * 77}, chunk, false);
  }
  // a large table: the BERT-Large shapes (385 tensors, 333,563,904 elements)
  std::vector<int64_t> bert = {30522LL * 1024};
  for (int b = 0; b < 24; ++b)
    for (int64_t n : {1024LL * 1024, 1024LL, 1024LL * 1024, 1024LL, 1024LL * 1024, 1024LL,
                      1024LL * 1024, 1024LL, 1024LL, 1024LL, 1024LL * 4096, 4096LL,
                      4096LL * 1024, 1024LL, 1024LL, 1024LL})
      bert.push_back(n);
  check_table(bert, 4096, false);
}

// table_sizes at the bounds: at most 2^30 - 1 chunks and fewer than 2^32
// work-items in a launch of the widest table kernel, running sums that
// would overflow int64, non-positive sizes, NULL, L < 1, bad chunks.
static void fuzz_table_sizes() {
  for (int32_t chunk : kChunks) {
    const int64_t max_n = ref_max_n(chunk, true);
    int64_t N = -1, K = -1;
    std::vector<int64_t> v = {max_n};
    EXPECT(table_sizes(v.data(), 1, chunk, &N, &K, "f") == ONEBIT_OK && N == max_n &&
               K == max_n / chunk,
           "exact bound refused at chunk %d", chunk);
    v = {max_n + 1};
    EXPECT(table_sizes(v.data(), 1, chunk, &N, &K, "f") == ONEBIT_EUNSUPPORTED, "bound + 1");
    v = {max_n - 5, 5};
    EXPECT(table_sizes(v.data(), 2, chunk, &N, &K, "f") == ONEBIT_OK, "split bound refused");
    v = {max_n - 5, 6};
    EXPECT(table_sizes(v.data(), 2, chunk, &N, &K, "f") == ONEBIT_EUNSUPPORTED, "split bound + 1");
    v = {INT64_MAX, INT64_MAX, INT64_MAX};
    EXPECT(table_sizes(v.data(), 3, chunk, &N, &K, "f") == ONEBIT_EUNSUPPORTED, "int64 max");
    v = {1LL << 62, 1LL << 62, 1LL << 62};
    EXPECT(table_sizes(v.data(), 3, chunk, &N, &K, "f") == ONEBIT_EUNSUPPORTED, "2^62 x 3");
    v = {5, 0, 7};
    EXPECT(table_sizes(v.data(), 3, chunk, &N, &K, "f") == ONEBIT_EINVAL, "zero size");
    v = {5, INT64_MIN, 7};
    EXPECT(table_sizes(v.data(), 3, chunk, &N, &K, "f") == ONEBIT_EINVAL, "negative size");
    EXPECT(table_sizes(v.data(), 0, chunk, &N, &K, "f") == ONEBIT_EINVAL, "L = 0");
    EXPECT(table_sizes(v.data(), -3, chunk, &N, &K, "f") == ONEBIT_EINVAL, "L < 0");
    EXPECT(table_sizes(nullptr, 1, chunk, &N, &K, "f") == ONEBIT_EINVAL, "NULL numels");
  }
  int64_t N, K;
  std::vector<int64_t> v = {100};
  for (int32_t c : {0, -4096, 32, 1, 1000, 3000, 1 << 25, 1 << 30, (1 << 24) + 64, 4097, 96,
                    INT32_MIN, INT32_MAX})
    EXPECT(table_sizes(v.data(), 1, c, &N, &K, "f") == ONEBIT_EUNSUPPORTED, "chunk %d", c);
  // random sizes near the bound against a 128-bit sum
  std::mt19937_64 r(2);
  for (int it = 0; it < 20000; ++it) {
    const int32_t chunk = kChunks[r() % kNChunks];
    const int L = 1 + (int)(r() % 6);
    std::vector<int64_t> n(L);
    for (int l = 0; l < L; ++l) {
      switch (r() % 4) {
        case 0: n[l] = (int64_t)(r() >> 1); break;                                  // anything
        case 1: n[l] = ref_max_n(chunk, true) / L + (int64_t)(r() % 64) - 32; break;  // near the bound
        case 2: n[l] = (int64_t)(r() % 1000) - 5; break;                            // small, some < 1
        default: n[l] = INT64_MAX - (int64_t)(r() % 3); break;
      }
    }
    i128 sum = 0;
    bool bad_size = false;
    for (int64_t x : n) {
      if (x < 1) bad_size = true;
      sum += x;
    }
    int expect;
    if (bad_size) {
      // the first non-positive size is reported unless the bound is passed before it
      i128 run = 0;
      expect = ONEBIT_EINVAL;
      for (int64_t x : n) {
        if (x < 1) break;
        run += x;
        if (run > (i128)ref_max_n(chunk, true)) {
          expect = ONEBIT_EUNSUPPORTED;
          break;
        }
      }
    } else {
      expect = sum > (i128)ref_max_n(chunk, true) ? ONEBIT_EUNSUPPORTED : ONEBIT_OK;
    }
    const int rc = table_sizes(n.data(), L, chunk, &N, &K, "f");
    EXPECT(rc == expect, "random sizes: rc %d expected %d", rc, expect);
    if (rc == ONEBIT_OK) EXPECT((i128)N == sum && (i128)K == (sum + chunk - 1) / chunk, "N or K");
  }
}

// ---------------------------------------------------------------------------
// scalar checks and byte counts
// ---------------------------------------------------------------------------
static void fuzz_scalars() {
  std::mt19937_64 r(3);
  const int64_t edges[] = {0, 1, 4095, 4096, 4097, INT64_MAX, INT64_MAX - 1, INT64_MIN, -1,
                           kMaxChunks * 1024, kMaxChunks * 1024 + 1, kMaxChunks * 16384,
                           kMaxChunks * 16384 + 1, kMaxChunks * (1LL << 24),
                           kMaxChunks * (1LL << 24) + 1};
  for (int it = 0; it < 200000; ++it) {
    const int64_t chunk = kChunks[r() % kNChunks];
    int64_t n;
    if (it < (int)(sizeof edges / sizeof edges[0])) n = edges[it];
    else if (r() % 2) n = (int64_t)r();
    else n = (int64_t)(r() % ((uint64_t)ref_max_n(chunk, false) + 2));
    const int rc = check_n(n, chunk, "f");
    const i128 k = n < 0 ? 0 : ((i128)n + chunk - 1) / chunk;
    const int expect =
        n < 0 ? ONEBIT_EINVAL : (ref_fits(k, (int32_t)chunk, false) ? ONEBIT_OK : ONEBIT_EUNSUPPORTED);
    EXPECT(rc == expect, "check_n(%lld, %lld) = %d, expected %d", (long long)n, (long long)chunk, rc,
           expect);
    if (rc == ONEBIT_OK) {
      EXPECT(chunks_of(n, chunk) == (int64_t)k, "chunks_of");
      const Bytes b(n, chunk);
      EXPECT((i128)b.elems == (i128)4 * n && (i128)b.words == 4 * (k * chunk / 32) &&
                 (i128)b.scales == 4 * k,
             "Bytes(%lld, %lld)", (long long)n, (long long)chunk);
    }
  }
  // the exact bound at every chunk size: four slots per thread, and two (the
  // 1-bit Adam warmup's layout at 4096)
  for (int32_t chunk : kChunks) {
    const int64_t n = ref_max_n(chunk, false);
    EXPECT(check_n(n, chunk, "f") == ONEBIT_OK, "check_n at the bound, chunk %d", chunk);
    EXPECT(check_n(n + 1, chunk, "f") == ONEBIT_EUNSUPPORTED, "check_n past the bound, chunk %d",
           chunk);
  }
  EXPECT(check_n(ref_max_n(4096, true), 4096, "f", 2) == ONEBIT_OK &&
             check_n(ref_max_n(4096, true) + 1, 4096, "f", 2) == ONEBIT_EUNSUPPORTED,
         "check_n with two slots per thread");
  EXPECT(ref_max_n(64, false) == 67108863LL * 64 && ref_max_n(4096, false) == 16777215LL * 4096 &&
             ref_max_n(1 << 20, false) == 16777215LL << 20,
         "reference bounds");
  for (int W = -3; W <= 20; ++W)
    EXPECT((check_W(W, "f") == ONEBIT_OK) == (W >= 1 && W <= 16), "check_W(%d)", W);
  EXPECT(check_W(INT32_MIN, "f") == ONEBIT_EUNSUPPORTED && check_W(INT32_MAX, "f") == ONEBIT_EUNSUPPORTED,
         "check_W extremes");
  // every power of two from 64 to 2^24, nothing else
  for (int32_t c = -70000; c <= 140000; ++c)
    EXPECT(chunk_supported(c) == (c == 64 || c == 128 || c == 256 || c == 512 || c == 1024 ||
                                  c == 2048 || c == 4096 || c == 8192 || c == 16384 ||
                                  c == 32768 || c == 65536 || c == 131072),
           "chunk_supported(%d)", c);
  for (int e = 17; e <= 30; ++e) {
    EXPECT(chunk_supported(1 << e) == (e <= 24), "chunk_supported(2^%d)", e);
    EXPECT(!chunk_supported((1 << e) + 64) && !chunk_supported((1 << e) - 64),
           "chunk_supported(2^%d +- 64)", e);
  }
  // error text is kept per thread and cleared by a success
  fail(ONEBIT_EINVAL, "msg %d", 7);
  EXPECT(last_error_slot() == "msg 7", "fail message");
  ok();
  EXPECT(last_error_slot().empty(), "ok clears");
  // long messages are cut, not overrun
  std::string big(2000, 'x');
  fail(ONEBIT_EINVAL, "%s", big.c_str());
  EXPECT(last_error_slot().size() == 511, "message length %zu", last_error_slot().size());
}

// ---------------------------------------------------------------------------
// overlap check
// ---------------------------------------------------------------------------
struct Ref {
  uint64_t p;
  int64_t bytes;
  bool w;
};

static int reference_spans(const std::vector<Ref>& v) {
  std::vector<Ref> s;
  for (const Ref& x : v)
    if (x.p && x.bytes > 0) s.push_back(x);
  if ((int)s.size() > Spans::kCap) return ONEBIT_EINVAL;
  for (const Ref& x : s)
    if ((i128)x.p + x.bytes >= ((i128)1 << 64)) return ONEBIT_EINVAL;  // end not representable
  for (size_t i = 0; i < s.size(); ++i)
    for (size_t j = i + 1; j < s.size(); ++j)
      if ((s[i].w || s[j].w) && (i128)s[i].p < (i128)s[j].p + s[j].bytes &&
          (i128)s[j].p < (i128)s[i].p + s[i].bytes)
        return ONEBIT_EINVAL;
  return ONEBIT_OK;
}

static void fuzz_spans() {
  std::mt19937_64 r(4);
  for (int it = 0; it < 100000; ++it) {
    const int n = (int)(r() % 12);
    std::vector<Ref> v;
    const bool high = r() % 8 == 0;  // near the top of the address space
    for (int i = 0; i < n; ++i) {
      Ref x;
      x.p = high ? UINT64_MAX - (r() % 4096) : (r() % 4096);
      if (r() % 16 == 0) x.p = 0;
      x.bytes = (int64_t)(r() % 600) - 20;
      if (r() % 32 == 0) x.bytes = INT64_MAX - (int64_t)(r() % 4);
      x.w = r() % 3 == 0;
      v.push_back(x);
    }
    Spans sp;
    for (int i = 0; i < n; ++i) sp.add(reinterpret_cast<const void*>(v[i].p), v[i].bytes, v[i].w, "a", i);
    const int rc = sp.check("f");
    const int expect = reference_spans(v);
    EXPECT(rc == expect, "spans: rc %d expected %d (%d arrays)", rc, expect, n);
  }
  // more arrays than the checker holds is an error, not a silent pass
  Spans sp;
  for (int i = 0; i < Spans::kCap + 1; ++i)
    sp.add(reinterpret_cast<const void*>((uintptr_t)(4096 + 64 * i)), 16, false, "a", i);
  EXPECT(sp.check("f") == ONEBIT_EINVAL, "capacity overflow passed");
  // workers: one gradient read by all is fine, one error written by two is not
  const void* g[3] = {reinterpret_cast<const void*>(4096), reinterpret_cast<const void*>(4096),
                      reinterpret_cast<const void*>(4096)};
  Spans a;
  a.add_workers(g, 3, 1024, false, "grads");
  EXPECT(a.check("f") == ONEBIT_OK, "shared read-only gradient refused");
  Spans b;
  b.add_workers(g, 3, 1024, true, "err_w");
  EXPECT(b.check("f") == ONEBIT_EINVAL && last_error_slot().find("err_w[1] overlaps err_w[0]") !=
                                               std::string::npos,
         "shared written error passed: %s", last_error_slot().c_str());
  Spans c;
  c.add_workers((const void* const*)nullptr, 3, 1024, true, "none");
  EXPECT(c.size() == 0 && c.check("f") == ONEBIT_OK, "NULL worker array");
}

// ---------------------------------------------------------------------------
// hyper-parameters
// ---------------------------------------------------------------------------
static onebit_hparams good_hp() {
  onebit_hparams h;
  std::memset(&h, 0, sizeof h);
  h.beta1 = 0.9f;
  h.beta2 = 0.999f;
  h.eta = 1e-8f;
  h.lr = 1e-3f;
  h.c_min = 0.01f;
  h.c_max = 10.0f;
  h.f_min = 0.5f;
  h.f_max = 4.0f;
  h.kappa = 0.1f;
  return h;
}

// Reference predicate, written from the documented domains.
static bool hp_valid(const onebit_hparams& h, bool allow_wd, int* code) {
  auto in01 = [](float b) { return b >= 0.0f && b < 1.0f; };
  const bool finite_eta = std::isfinite(h.eta);
  bool v = in01(h.beta1) && in01(h.beta2) && finite_eta && h.eta >= 0.0f && std::isfinite(h.lr) &&
           std::isfinite(h.weight_decay) && h.weight_decay >= 0.0f && std::isfinite(h.c_min) &&
           h.c_min >= 0.0f && !std::isnan(h.c_max) && h.c_max >= h.c_min &&
           std::isfinite(h.f_min) && h.f_min >= 0.0f && !std::isnan(h.f_max) &&
           h.f_max >= h.f_min && std::isfinite(h.kappa) && h.kappa >= 0.0f &&
           (h.rho_mode == 0 || h.rho_mode == 1) && in01(h.c_avg_decay) && h.bias_step >= 0;
  *code = ONEBIT_EINVAL;
  if (v && !allow_wd && h.weight_decay != 0.0f) {
    *code = ONEBIT_EUNSUPPORTED;
    return false;
  }
  return v;
}

static void fuzz_hparams() {
  EXPECT(check_hparams(nullptr, "f") == ONEBIT_EINVAL, "NULL hp");
  onebit_hparams h = good_hp();
  EXPECT(check_hparams(&h, "f") == ONEBIT_OK, "defaults refused: %s", last_error_slot().c_str());
  const float inf = std::numeric_limits<float>::infinity();
  const float nan = std::numeric_limits<float>::quiet_NaN();
  struct Case {
    float onebit_hparams::*f;
    float val;
    bool valid;
    const char* what;
  } cases[] = {
      {&onebit_hparams::beta1, 1.0f, false, "beta1 = 1"},
      {&onebit_hparams::beta1, -0.1f, false, "beta1 < 0"},
      {&onebit_hparams::beta1, nan, false, "beta1 NaN"},
      {&onebit_hparams::beta1, 0.0f, true, "beta1 = 0"},
      {&onebit_hparams::beta1, 0.99999994f, true, "beta1 just below 1"},
      {&onebit_hparams::beta2, 1.0f, false, "beta2 = 1"},
      {&onebit_hparams::beta2, 1.5f, false, "beta2 > 1"},
      {&onebit_hparams::beta2, nan, false, "beta2 NaN"},
      {&onebit_hparams::eta, -1e-8f, false, "eta < 0"},
      {&onebit_hparams::eta, nan, false, "eta NaN"},
      {&onebit_hparams::eta, inf, false, "eta inf"},
      {&onebit_hparams::eta, 0.0f, true, "eta = 0"},
      {&onebit_hparams::lr, inf, false, "lr inf"},
      {&onebit_hparams::lr, -inf, false, "lr -inf"},
      {&onebit_hparams::lr, nan, false, "lr NaN"},
      {&onebit_hparams::lr, -1e-3f, true, "lr < 0 (finite)"},
      {&onebit_hparams::weight_decay, -0.1f, false, "weight_decay < 0"},
      {&onebit_hparams::weight_decay, inf, false, "weight_decay inf"},
      {&onebit_hparams::c_min, 20.0f, false, "c_min > c_max"},
      {&onebit_hparams::c_min, -1.0f, false, "c_min < 0"},
      {&onebit_hparams::c_min, nan, false, "c_min NaN"},
      {&onebit_hparams::c_min, 10.0f, true, "c_min = c_max"},
      {&onebit_hparams::c_max, inf, true, "c_max inf"},
      {&onebit_hparams::c_max, nan, false, "c_max NaN"},
      {&onebit_hparams::c_max, 0.001f, false, "c_max < c_min"},
      {&onebit_hparams::f_min, 5.0f, false, "f_min > f_max"},
      {&onebit_hparams::f_min, -0.5f, false, "f_min < 0"},
      {&onebit_hparams::f_min, nan, false, "f_min NaN"},
      {&onebit_hparams::f_max, inf, true, "f_max inf"},
      {&onebit_hparams::f_max, nan, false, "f_max NaN"},
      {&onebit_hparams::kappa, -0.1f, false, "kappa < 0"},
      {&onebit_hparams::kappa, inf, false, "kappa inf"},
      {&onebit_hparams::kappa, nan, false, "kappa NaN"},
      {&onebit_hparams::kappa, 0.0f, true, "kappa = 0"},
      {&onebit_hparams::c_avg_decay, 1.0f, false, "c_avg_decay = 1"},
      {&onebit_hparams::c_avg_decay, -0.5f, false, "c_avg_decay < 0"},
  };
  for (const Case& c : cases) {
    onebit_hparams x = good_hp();
    x.*(c.f) = c.val;
    const int rc = check_hparams(&x, "f");
    EXPECT((rc == ONEBIT_OK) == c.valid, "%s: rc %d", c.what, rc);
    if (!c.valid) EXPECT(rc == ONEBIT_EINVAL && !last_error_slot().empty(), "%s: code", c.what);
  }
  h = good_hp();
  h.rho_mode = 2;
  EXPECT(check_hparams(&h, "f") == ONEBIT_EINVAL, "rho_mode 2");
  h = good_hp();
  h.bias_step = -1;
  EXPECT(check_hparams(&h, "f") == ONEBIT_EINVAL, "bias_step -1");
  h = good_hp();
  h.weight_decay = 0.01f;
  EXPECT(check_hparams(&h, "f", false) == ONEBIT_EUNSUPPORTED, "wd in Adam mode");
  // an all-zero struct is valid (every bound is met with equality)
  std::memset(&h, 0, sizeof h);
  EXPECT(check_hparams(&h, "f") == ONEBIT_OK, "zero struct refused: %s", last_error_slot().c_str());
  // random structs against the reference predicate
  std::mt19937_64 r(5);
  const float pool[] = {0.0f, -0.0f, 0.5f, 0.9f, 0.999f, 1.0f, 1.5f, -0.1f, 10.0f, 1e-8f,
                        inf, -inf, nan, 1e30f, 4.0f, 0.01f};
  for (int it = 0; it < 300000; ++it) {
    onebit_hparams x = good_hp();
    float* fields[] = {&x.beta1, &x.beta2, &x.eta, &x.lr, &x.weight_decay, &x.c_min,
                       &x.c_max, &x.f_min, &x.f_max, &x.kappa, &x.c_avg_decay};
    const int nf = (int)(sizeof fields / sizeof fields[0]);
    const int changes = 1 + (int)(r() % 3);
    for (int i = 0; i < changes; ++i) *fields[r() % nf] = pool[r() % (sizeof pool / sizeof pool[0])];
    if (r() % 10 == 0) x.rho_mode = (int32_t)(r() % 4) - 1;
    if (r() % 10 == 0) x.bias_step = (int32_t)(r() % 5) - 2;
    const bool allow_wd = r() % 2;
    int code = 0;
    const bool valid = hp_valid(x, allow_wd, &code);
    const int rc = check_hparams(&x, "f", allow_wd);
    EXPECT(valid ? rc == ONEBIT_OK : rc == code, "random hparams: rc %d valid %d code %d", rc,
           (int)valid, code);
  }
}

// ---------------------------------------------------------------------------
// workspace layout
// ---------------------------------------------------------------------------
static void fuzz_workspace() {
  std::mt19937_64 r(6);
  for (int it = 0; it < 100000; ++it) {
    const int64_t S = (int64_t)(r() % ((uint64_t)INT32_MAX + 1));
    const int32_t L = (int32_t)(r() % ((uint64_t)INT32_MAX + 1));
    const size_t total = ws_bytes(S, L);
    const WsOffsets o = ws_offsets(S);
    // parts: seg_x [0, 8S), seg_u [o.seg_u, +8S), c_layer [o.c_layer, +4L);
    // 256-byte aligned, disjoint, inside the total
    EXPECT(o.seg_x % 256 == 0 && o.seg_u % 256 == 0 && o.c_layer % 256 == 0, "alignment");
    EXPECT(o.seg_x + 8 * (size_t)S <= o.seg_u && o.seg_u + 8 * (size_t)S <= o.c_layer &&
               o.c_layer + 4 * (size_t)L <= total,
           "overlap or overrun at S %lld L %d", (long long)S, L);
    EXPECT(o.seg_max == o.seg_x && 4 * (size_t)S <= o.seg_u, "seg_max inside seg_x");
    EXPECT(total < 8 * (size_t)S + 8 * (size_t)S + 4 * (size_t)L + 3 * 256, "padding");
  }
}

int main() {
  fuzz_tables();
  fuzz_table_sizes();
  fuzz_scalars();
  fuzz_spans();
  fuzz_hparams();
  fuzz_workspace();
  if (g_fail) {
    std::printf("%d failures\n", g_fail);
    return 1;
  }
  std::printf("host check ok\n");
  return 0;
}
