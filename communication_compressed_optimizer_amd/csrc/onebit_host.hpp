// Host-side logic of libonebit.so that needs no GPU: error reporting,
// argument and hyper-parameter checks, the overlap check of a call's arrays,
// byte sizes, the workspace layout and the construction of the tensor table.
//
// This header includes no HIP header, so the same code is compiled into the
// library (by onebit.hip) and into a plain C++ test driver built with
// AddressSanitizer and UndefinedBehaviorSanitizer, which fuzzes it on the
// CPU against brute-force references.
#pragma once

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <limits>
#include <new>
#include <string>
#include <vector>

#include "onebit.h"

namespace onebit_host {

// ---------------------------------------------------------------------------
// error reporting: the message of the calling thread's last failure
// ---------------------------------------------------------------------------
inline std::string& last_error_slot() {
  static thread_local std::string s;
  return s;
}

inline int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
inline int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  last_error_slot() = buf;
  return code;
}

inline int ok() {
  last_error_slot().clear();
  return ONEBIT_OK;
}

// ---------------------------------------------------------------------------
// scalar checks
// ---------------------------------------------------------------------------
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Chunks of 64 .. 2^24 elements, powers of two.
inline bool chunk_supported(int32_t c) { return c >= 64 && c <= (1 << 24) && (c & (c - 1)) == 0; }

inline size_t round256(size_t b) { return (b + 255) & ~size_t(255); }

constexpr int kMaxWorkers = ONEBIT_MAX_WORKERS;

// Chunk counts beyond this are refused at any chunk size (chunk and segment
// indices are 32-bit).
constexpr int64_t kMaxChunks = INT32_MAX / 2;

// Threads per chunk of a launch that lays `slots` float4 slots per thread,
// one workgroup per chunk: one 64-wide wave below 1024 elements (the padded
// geometry), chunk / (4 * slots) up to 16384, and 256 above (a workgroup
// that walks the chunk in 4096-element blocks).
constexpr int64_t chunk_threads(int64_t chunk, int64_t slots) {
  return chunk < 1024 ? 64 : (chunk > 16384 ? 256 : chunk / (4 * slots));
}

// Float4 slots per thread of the narrowest layout a kernel on a layer table
// takes at this chunk size: two for the warmup passes at 4096, else four.
// onebit.hip checks its launch geometries against it at compile time.
constexpr int64_t table_slots(int64_t chunk) { return chunk == 4096 ? 2 : 4; }

// Chunks one launch of that layout may cover.  A dispatch counts its grid in
// work-items, 32 bits wide, so chunks * chunk_threads must stay below 2^32;
// that binds only below 1024 elements (at 64: fewer than 2^32 elements).
constexpr int64_t max_chunks(int64_t chunk, int64_t slots = 4) {
  return (int64_t)UINT32_MAX / chunk_threads(chunk, slots) < kMaxChunks
             ? (int64_t)UINT32_MAX / chunk_threads(chunk, slots)
             : kMaxChunks;
}

// ceil(n / chunk) for n >= 0, chunk >= 1, without the overflow of n + chunk - 1.
inline int64_t chunks_of(int64_t n, int64_t chunk) { return n / chunk + (n % chunk != 0); }

// n >= 0 (EINVAL) and at most max_chunks(chunk, slots) chunks (EUNSUPPORTED).
inline int check_n(int64_t n, int64_t chunk, const char* fn, int64_t slots = 4) {
  if (n < 0) return fail(ONEBIT_EINVAL, "%s: n < 0", fn);
  if (chunks_of(n, chunk) > max_chunks(chunk, slots))
    return fail(ONEBIT_EUNSUPPORTED, "%s: n too large (at most %lld chunks of %lld)", fn,
                (long long)max_chunks(chunk, slots), (long long)chunk);
  return ONEBIT_OK;
}

inline int check_W(int32_t W, const char* fn) {
  if (W < 1 || W > kMaxWorkers)
    return fail(ONEBIT_EUNSUPPORTED, "%s: W = %d outside [1, %d]", fn, W, kMaxWorkers);
  return ONEBIT_OK;
}

// The hyper-parameters' domains ("1-bit LAMB", Background on LAMB: beta1 and
// beta2 are decay factors, eta is an additive constant that keeps the
// denominator away from 0, clip(x, a, b) = min{max{x, a}, b}).  Every field
// is checked by every entry point that takes hp, whether it uses the field
// or not, so that a struct is valid or invalid as a whole (EINVAL), before
// the 1-bit Adam mode's refusal of weight decay (EUNSUPPORTED):
//   beta1, beta2 in [0, 1) (beta1 = 1 would divide the reconstructed
//   gradient by 1 - beta1 = 0); eta >= 0 and finite; lr finite;
//   weight_decay >= 0 and finite; 0 <= c_min <= c_max and 0 <= f_min <=
//   f_max (the upper bounds may be +inf: no clip); kappa >= 0 and finite;
//   rho_mode one of the two readings; c_avg_decay in [0, 1); bias_step >= 0.
// allow_wd: weight decay is a variant of the LAMB entry points only.
inline int check_hparams(const onebit_hparams* hp, const char* fn, bool allow_wd = true) {
  if (!hp) return fail(ONEBIT_EINVAL, "%s: hp is NULL", fn);
  if (!(hp->beta1 >= 0.0f && hp->beta1 < 1.0f))
    return fail(ONEBIT_EINVAL, "%s: beta1 = %g outside [0, 1)", fn, (double)hp->beta1);
  if (!(hp->beta2 >= 0.0f && hp->beta2 < 1.0f))
    return fail(ONEBIT_EINVAL, "%s: beta2 = %g outside [0, 1)", fn, (double)hp->beta2);
  if (!(std::isfinite(hp->eta) && hp->eta >= 0.0f))
    return fail(ONEBIT_EINVAL, "%s: eta = %g must be finite and >= 0", fn, (double)hp->eta);
  if (!std::isfinite(hp->lr)) return fail(ONEBIT_EINVAL, "%s: lr is not finite", fn);
  if (!std::isfinite(hp->weight_decay) || hp->weight_decay < 0.0f)
    return fail(ONEBIT_EINVAL, "%s: weight_decay must be finite and >= 0", fn);
  if (!(hp->c_min >= 0.0f && std::isfinite(hp->c_min) && hp->c_max >= hp->c_min))
    return fail(ONEBIT_EINVAL, "%s: clip bounds need 0 <= c_min <= c_max (c_min = %g, c_max = %g)",
                fn, (double)hp->c_min, (double)hp->c_max);
  if (!(hp->f_min >= 0.0f && std::isfinite(hp->f_min) && hp->f_max >= hp->f_min))
    return fail(ONEBIT_EINVAL,
                "%s: soft thresholds need 0 <= f_min <= f_max (f_min = %g, f_max = %g)", fn,
                (double)hp->f_min, (double)hp->f_max);
  if (!(std::isfinite(hp->kappa) && hp->kappa >= 0.0f))
    return fail(ONEBIT_EINVAL, "%s: kappa = %g must be finite and >= 0", fn, (double)hp->kappa);
  if (hp->rho_mode != ONEBIT_RHO_MAX && hp->rho_mode != ONEBIT_RHO_NORM_RATIO)
    return fail(ONEBIT_EINVAL, "%s: rho_mode %d is not ONEBIT_RHO_MAX or ONEBIT_RHO_NORM_RATIO", fn,
                hp->rho_mode);
  if (!(hp->c_avg_decay >= 0.0f && hp->c_avg_decay < 1.0f))
    return fail(ONEBIT_EINVAL, "%s: c_avg_decay must be in [0, 1)", fn);
  if (hp->bias_step < 0) return fail(ONEBIT_EINVAL, "%s: bias_step < 0", fn);
  // a valid struct that asks for what the mode does not support
  if (!allow_wd && hp->weight_decay != 0.0f)
    return fail(ONEBIT_EUNSUPPORTED, "%s: weight_decay must be 0 in the 1-bit Adam mode", fn);
  return ONEBIT_OK;
}

// ---------------------------------------------------------------------------
// byte ranges of one call's arrays
// ---------------------------------------------------------------------------
// The kernels access a call's arrays through restrict-qualified pointers, so
// an array the call writes must not overlap any other array of the call;
// read-only arrays may overlap each other (one gradient buffer passed for
// several workers, say).  An array whose one-past-the-end address is not
// representable (its range reaches the end of the address space) is refused
// too, so that the interval arithmetic below cannot wrap.
class Spans {
 public:
  void add(const void* p, int64_t bytes, bool written, const char* name, int idx = -1) {
    if (!p || bytes <= 0) return;
    if (n_ == kCap) {
      overflow_ = true;
      return;
    }
    s_[n_++] = {reinterpret_cast<uintptr_t>(p), (uintptr_t)bytes, written, name, idx};
  }
  // Every array of W workers, given as a host array of pointers (or NULL).
  template <typename T>
  void add_workers(T const* arr, int W, int64_t bytes, bool written, const char* name) {
    if (arr)
      for (int w = 0; w < W; ++w) add(arr[w], bytes, written, name, w);
  }
  int check(const char* fn) const {
    if (overflow_) return fail(ONEBIT_EINVAL, "%s: more than %d arrays to check", fn, kCap);
    for (int i = 0; i < n_; ++i)
      if (s_[i].bytes > std::numeric_limits<uintptr_t>::max() - s_[i].p)  // end >= 2^64
        return fail(ONEBIT_EINVAL, "%s: %s runs past the end of the address space", fn,
                    label(s_[i]).c_str());
    for (int i = 0; i < n_; ++i)
      for (int j = i + 1; j < n_; ++j) {
        const S& a = s_[i];
        const S& b = s_[j];
        if ((a.w || b.w) && a.p < b.p + b.bytes && b.p < a.p + a.bytes) {
          const S& wr = b.w ? b : a;  // the written one is named first
          const S& other = b.w ? a : b;
          return fail(ONEBIT_EINVAL, "%s: %s overlaps %s", fn, label(wr).c_str(),
                      label(other).c_str());
        }
      }
    return ONEBIT_OK;
  }
  int size() const { return n_; }

  // four worker arrays of up to kMaxWorkers entries plus a dozen others
  static constexpr int kCap = 4 * kMaxWorkers + 16;

 private:
  struct S {
    uintptr_t p, bytes;
    bool w;
    const char* name;
    int idx;
  };
  static std::string label(const S& s) {
    return s.idx < 0 ? std::string(s.name) : std::string(s.name) + "[" + std::to_string(s.idx) + "]";
  }
  S s_[kCap];
  int n_ = 0;
  bool overflow_ = false;
};

// Bytes of a buffer's arrays: n elements in chunks of `chunk` (n within
// check_n's bound, so nothing here overflows).
struct Bytes {
  int64_t elems, words, scales;
  Bytes(int64_t n, int64_t chunk) {
    const int64_t K = chunks_of(n, chunk);
    elems = 4 * n;
    words = 4 * (K * chunk / 32);
    scales = 4 * K;
  }
};

// ---------------------------------------------------------------------------
// the tensor table
// ---------------------------------------------------------------------------
// L tensors of numels[l] elements concatenated in order; chunk k is the
// elements [k*chunk, min((k+1)*chunk, N)).  A (chunk, tensor) segment is a
// pair whose ranges intersect; segments are numbered chunk by chunk, and
// within a chunk tensor by tensor.
struct HostTable {
  int32_t L = 0;
  int32_t chunk = 0;
  int64_t N = 0;
  int64_t K = 0;
  int64_t S = 0;               // number of segments
  std::vector<int64_t> off;    // [L+1] flat offset of each tensor
  std::vector<int32_t> l0;     // [K] first tensor chunk k touches
  std::vector<int32_t> l1;     // [K] last tensor chunk k touches
  std::vector<int32_t> seg;    // [K] number of segment (k, l0[k])
  std::vector<int32_t> lseg;   // [L+1] segments of tensor l are [lseg[l], lseg[l+1])
};

// Checks the sizes and returns N and K without building anything: EINVAL for
// a NULL array, L < 1 or a tensor of fewer than 1 element; EUNSUPPORTED for a
// chunk that is not a power of two in [64, 2^24] or more than
// max_chunks(chunk, table_slots(chunk)) chunks in all.  The running sum is
// bounded before each add, so it cannot overflow.
inline int table_sizes(const int64_t* numels, int32_t L, int32_t chunk, int64_t* N, int64_t* K,
                       const char* fn) {
  if (!numels) return fail(ONEBIT_EINVAL, "%s: NULL argument", fn);
  if (L < 1) return fail(ONEBIT_EINVAL, "%s: L = %d < 1", fn, L);
  if (!chunk_supported(chunk))
    return fail(ONEBIT_EUNSUPPORTED, "%s: chunk %d is not a power of two in [64, 2^24]", fn,
                chunk);
  const int64_t max_n = max_chunks(chunk, table_slots(chunk)) * chunk;
  int64_t n = 0;
  for (int32_t l = 0; l < L; ++l) {
    if (numels[l] < 1)
      return fail(ONEBIT_EINVAL, "%s: numels[%d] = %lld < 1", fn, l, (long long)numels[l]);
    if (numels[l] > max_n - n) return fail(ONEBIT_EUNSUPPORTED, "%s: too many chunks", fn);
    n += numels[l];
  }
  *N = n;
  *K = chunks_of(n, chunk);
  return ONEBIT_OK;
}

// Builds the table's host arrays (table_sizes' errors; ENOMEM when a host
// allocation fails; EUNSUPPORTED beyond 2^31 - 1 segments).
inline int build_table(const int64_t* numels, int32_t L, int32_t chunk, HostTable& t,
                       const char* fn) {
  int64_t N = 0, K = 0;
  if (int rc = table_sizes(numels, L, chunk, &N, &K, fn)) return rc;
  try {
    t.off.assign((size_t)L + 1, 0);
    for (int32_t l = 0; l < L; ++l) t.off[l + 1] = t.off[l] + numels[l];
    t.l0.assign((size_t)K, 0);
    t.l1.assign((size_t)K, 0);
    t.seg.assign((size_t)K, 0);
    t.lseg.assign((size_t)L + 1, 0);
  } catch (const std::bad_alloc&) {
    return fail(ONEBIT_ENOMEM, "%s: host allocation failed", fn);
  }
  int64_t S = 0;
  int32_t l = 0;
  for (int64_t k = 0; k < K; ++k) {
    const int64_t first = k * chunk;
    const int64_t last = (k + 1) * chunk < N ? (k + 1) * chunk - 1 : N - 1;
    while (t.off[l + 1] <= first) ++l;
    t.l0[k] = l;
    int32_t e = l;
    while (t.off[e + 1] <= last) ++e;
    t.l1[k] = e;
    if (S > INT32_MAX) return fail(ONEBIT_EUNSUPPORTED, "%s: too many segments", fn);
    t.seg[k] = (int32_t)S;
    S += e - l + 1;
  }
  if (S > INT32_MAX) return fail(ONEBIT_EUNSUPPORTED, "%s: too many segments", fn);
  for (int32_t i = 0; i < L; ++i) {
    const int64_t k = t.off[i] / chunk;
    t.lseg[i] = t.seg[k] + (i - t.l0[k]);
  }
  t.lseg[L] = (int32_t)S;
  t.L = L;
  t.chunk = chunk;
  t.N = N;
  t.K = K;
  t.S = S;
  return ONEBIT_OK;
}

// ---------------------------------------------------------------------------
// workspace layout
// ---------------------------------------------------------------------------
// [seg_x: S doubles][seg_u: S doubles][c_layer: L floats], each part rounded
// up to 256 bytes.  The warmup keeps the per-segment sums of x^2 and u^2
// there; the compression step reuses the first S floats as the per-segment
// maxima, or (norm-ratio rescale) seg_x and seg_u for its double sums.
inline size_t ws_bytes(int64_t S, int32_t L) {
  return 2 * round256(sizeof(double) * (size_t)S) + round256(sizeof(float) * (size_t)L);
}

struct WsOffsets {
  size_t seg_x, seg_u, seg_max, c_layer;
};

inline WsOffsets ws_offsets(int64_t S) {
  WsOffsets o;
  o.seg_x = 0;
  o.seg_u = round256(sizeof(double) * (size_t)S);
  o.seg_max = 0;
  o.c_layer = 2 * round256(sizeof(double) * (size_t)S);
  return o;
}

}  // namespace onebit_host
