// libonebit_ceiling.so: pure-traffic kernels that measure what the HBM of
// the machine in hand sustains for the access patterns of the optimizer's
// kernels, as a practical ceiling beside the 8 TB/s peak.  They are
// measurement tools, not part of the optimizer: no entry point of
// libonebit.so calls them.
//
// They use the loads, stores, slot layout and launch shape of the step's
// kernels (onebit_kernels.hpp: one workgroup of 256 threads per chunk of
// 4096 elements, four float4 slots per thread, streaming accesses) and do
// almost no arithmetic:
//   onebit_ceiling_read    reads n floats (one word per workgroup written);
//   onebit_ceiling_copy    reads n floats and writes them to another buffer;
//   onebit_ceiling_phase1  the stream set of the compression step's first
//       phase on n elements and W workers: m read; per worker the gradient
//       and the error read, the error written back, the sign words written,
//       with one workgroup barrier per worker; the server error read and
//       written with a barrier; v_fresh and v_frozen read and v_fresh
//       written; the server's sign words written.  Its loads alone, or its
//       stores alone, and a cap on the workgroups per CU, can be asked for,
//       to see what the mix of reads and writes and the number of chunks in
//       flight cost.
// The written element arrays receive their own bits XOR `key`: with key = 0
// every state array keeps its value bit for bit, so the kernels can run on
// a step's real buffers (only the sign words, outputs of every step, are
// overwritten).  Only whole chunks are touched: n is rounded down to a
// multiple of 4096.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "onebit_kernels.hpp"

using namespace onebit;

namespace {

constexpr int C = 4096;
constexpr int T = C / 16;  // 256 threads, four float4 slots each

__device__ __forceinline__ void xor_slots(Slots& s, uint32_t key) {
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) s[a][c] = __uint_as_float(__float_as_uint(s[a][c]) ^ key);
}

__device__ __forceinline__ float slot_sum(const Slots& s) {
  float t = 0.0f;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) t = t + s[a][c];
  return t;
}

// One value per thread through LDS and a barrier, as a chunk reduction's
// cross-wave exchange does; returns a value that depends on another wave.
__device__ __forceinline__ float exchange(float v, float* lds, int& parity) {
  float* buf = lds + parity * T;
  parity ^= 1;
  buf[threadIdx.x] = v;
  __syncthreads();
  return buf[(threadIdx.x + 64) & (T - 1)];
}

// The word a group of eight lanes stores, made from a value of the chunk.
__device__ __forceinline__ void store_words(uint32_t* __restrict__ words, int64_t k, float v) {
  const int t = threadIdx.x;
  if ((t & 7) == 0) {
#pragma unroll
    for (int a = 0; a < 4; ++a) words[k * (C / 32) + ((t + T * a) >> 3)] = __float_as_uint(v) + a;
  }
}

__global__ void __launch_bounds__(T, 6)
k_ceiling_read(const float* __restrict__ in, float* __restrict__ sink) {
  Slots s;
  load_chunk<C, false, true>(in, (int64_t)blockIdx.x * C, C, s);
  const float v = slot_sum(s);
  if (v == 1.2345f) sink[blockIdx.x] = v;  // practically never: keeps the loads
}

__global__ void __launch_bounds__(T, 6)
k_ceiling_copy(const float* __restrict__ in, float* __restrict__ out) {
  Slots s;
  load_chunk<C, false, true>(in, (int64_t)blockIdx.x * C, C, s);
  store_chunk<C, false, true>(out, (int64_t)blockIdx.x * C, C, s);
}

struct PatternArgs {
  const float* g[kMaxWorkers];
  float* e[kMaxWorkers];
  uint32_t* bits[kMaxWorkers];
};

// MODE 0: the full stream set; 1: its loads only (the stores are kept out
// by a practically never true condition); 2: its stores only (the values
// come from the chunk index, not from memory, so the written arrays do NOT
// keep their contents).
template <int MODE>
__device__ __forceinline__ void pattern_load(const float* __restrict__ p, int64_t base, Slots& s,
                                             float salt) {
  if constexpr (MODE == 2) {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) s[a][c] = salt + (float)(a * 4 + c);
  } else {
    load_chunk<C, false, true>(p, base, C, s);
  }
}

template <int MODE>
__device__ __forceinline__ void pattern_store(float* __restrict__ p, int64_t base, const Slots& s) {
  if constexpr (MODE == 1) {
    if (s[0][0] == 1.2345f && s[3][3] == -1.2345f) p[base] = s[1][1];
  } else {
    store_chunk<C, false, true>(p, base, C, s);
  }
}

template <int MODE>
__global__ void __launch_bounds__(T, 6)
k_ceiling_phase1(int W, PatternArgs pa, const float* __restrict__ m, float* __restrict__ err_s,
                 const float* __restrict__ v_frozen, float* __restrict__ v_fresh,
                 uint32_t* __restrict__ bits_s, uint32_t key) {
  __shared__ float lds[2 * T];
  int parity = 0;
  const int64_t k = blockIdx.x;
  const int64_t base = k * C;
  const float salt = (float)(k & 1023);
  Slots mm;
  pattern_load<MODE>(m, base, mm, salt);
  float acc = slot_sum(mm);
  for (int w = 0; w < W; ++w) {
    Slots g, e;
    pattern_load<MODE>(pa.g[w], base, g, salt + (float)w);
    pattern_load<MODE>(pa.e[w], base, e, salt - (float)w);
    const float r = exchange(slot_sum(g) + slot_sum(e), lds, parity);
    acc = acc + r;
    xor_slots(e, key);
    pattern_store<MODE>(pa.e[w], base, e);
    if (pa.bits[w]) {
      if constexpr (MODE == 1) {
        if (r == 1.2345f) pa.bits[w][k] = 1u;
      } else {
        store_words(pa.bits[w], k, r);
      }
    }
  }
  Slots y;
  pattern_load<MODE>(err_s, base, y, salt * 0.5f);
  acc = acc + exchange(slot_sum(y), lds, parity);
  xor_slots(y, key);
  pattern_store<MODE>(err_s, base, y);
  if constexpr (MODE == 1) {
    if (acc == 1.2345f) bits_s[k] = 1u;
  } else {
    store_words(bits_s, k, acc);
  }
  Slots vf, vz;
  pattern_load<MODE>(v_fresh, base, vf, salt * 0.25f);
  pattern_load<MODE>(v_frozen, base, vz, salt * 0.125f);
  const float q = slot_sum(vz);
  xor_slots(vf, key ^ (q == 1.2345f ? 1u : 0u));  // depends on v_frozen
  pattern_store<MODE>(v_fresh, base, vf);
}

int launched() { return hipGetLastError() == hipSuccess ? 0 : 4; }

}  // namespace

extern "C" {

// n floats read (n rounded down to whole chunks of 4096); sink: n/4096
// floats, written only for a practically impossible chunk sum.  Returns 0,
// 1 (bad argument) or 4 (launch failed).
int onebit_ceiling_read(int64_t n, const float* in, float* sink, void* stream) {
  if (n < 0 || !in || !sink) return 1;
  const int64_t K = n / C;
  if (K == 0) return 0;
  if (K > INT32_MAX / 2) return 1;
  hipLaunchKernelGGL(k_ceiling_read, dim3((unsigned)K), dim3(T), 0, (hipStream_t)stream, in, sink);
  return launched();
}

// out[i] = in[i] for the n floats (rounded down to whole chunks).
int onebit_ceiling_copy(int64_t n, const float* in, float* out, void* stream) {
  if (n < 0 || !in || !out) return 1;
  const int64_t K = n / C;
  if (K == 0) return 0;
  if (K > INT32_MAX / 2) return 1;
  hipLaunchKernelGGL(k_ceiling_copy, dim3((unsigned)K), dim3(T), 0, (hipStream_t)stream, in, out);
  return launched();
}

// The stream set of the compression step's first phase (see the file
// comment).  g, e: host arrays of W device pointers to n floats; bits_w: a
// host array of W device pointers to n/32 words, or NULL (or NULL entries);
// m, v_frozen: n floats read; err_s, v_fresh: n floats read and written
// back XOR key; bits_s: n/32 words written.
// mode 0: the full set; 1: its loads only; 2: its stores only, with values
// made up from the chunk index (the written arrays then lose their
// contents).  lds_bytes > 0 gives every workgroup that much dynamic LDS,
// which caps how many run on a CU at once (160 KiB per CU).
int onebit_ceiling_phase1(int64_t n, int32_t W, const float* m, const float* const* g,
                          float* const* e, uint32_t* const* bits_w, float* err_s,
                          const float* v_frozen, float* v_fresh, uint32_t* bits_s, uint32_t key,
                          int32_t mode, int32_t lds_bytes, void* stream) {
  if (n < 0 || W < 1 || W > kMaxWorkers || !m || !g || !e || !err_s || !v_frozen || !v_fresh ||
      !bits_s || mode < 0 || mode > 2 || lds_bytes < 0 || lds_bytes > 150 * 1024)
    return 1;
  PatternArgs pa{};
  for (int w = 0; w < W; ++w) {
    if (!g[w] || !e[w]) return 1;
    pa.g[w] = g[w];
    pa.e[w] = e[w];
    pa.bits[w] = bits_w ? bits_w[w] : nullptr;
  }
  const int64_t K = n / C;
  if (K == 0) return 0;
  if (K > INT32_MAX / 2) return 1;
  hipStream_t st = (hipStream_t)stream;
  const dim3 grid((unsigned)K), block(T);
  if (mode == 0)
    hipLaunchKernelGGL(k_ceiling_phase1<0>, grid, block, lds_bytes, st, (int)W, pa, m, err_s,
                       v_frozen, v_fresh, bits_s, key);
  else if (mode == 1)
    hipLaunchKernelGGL(k_ceiling_phase1<1>, grid, block, lds_bytes, st, (int)W, pa, m, err_s,
                       v_frozen, v_fresh, bits_s, key);
  else
    hipLaunchKernelGGL(k_ceiling_phase1<2>, grid, block, lds_bytes, st, (int)W, pa, m, err_s,
                       v_frozen, v_fresh, bits_s, key);
  return launched();
}

}  // extern "C"
