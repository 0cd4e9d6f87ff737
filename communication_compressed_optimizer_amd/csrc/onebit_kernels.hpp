// HIP kernels of the 1-bit LAMB step for gfx950 (CDNA4, 64-wide waves), and
// of the 1-bit Adam mode and the SLAMB-style sparse stage built on the same
// pieces.
//
// Every kernel that touches chunks runs one workgroup per chunk of C
// elements with T = C/(4*SPT) threads (SPT = 4 float4 slots per thread from
// 1024 elements up unless a kernel says otherwise: T = C/16); thread t owns
// the slots p = t + T*k (k = 0..SPT-1) of its chunk, i.e. chunk elements
// 4p..4p+3.  The loads and stores of a wave are therefore 64 consecutive
// float4 (1 KiB) per slot: fully coalesced dwordx4 traffic.  Below 1024
// elements a chunk takes one wave: two slots per thread at 512, one at 256,
// and the chunks of 128 and 64 elements lie in the first 32 or 16 lanes of
// a one-slot wave (struct Geo below).
//
// Chunk scale.  The sum of squares of a chunk is the stride-halving tree
// t[j] += t[j+h], h = C/2, ..., 1 (zero past the last valid element), which
// fixes one rounding order so that scales, and through error feedback every
// later sign, are reproducible bit for bit.  With the slot layout above the
// levels h >= 4 act on the float4 slot index p with strides P/2..1
// (P = C/4) independently per component; strides 2T and T pair a thread's
// own slots, strides T/2..64 pair waves (through LDS), strides 32..1 pair
// lanes (lane swaps and DPP row shifts), and the last two levels (h = 2, 1)
// combine the four components: (c0 + c2) + (c1 + c3).
//
// Packed signs.  Element 4p+c sits in word p/8 at bit 4(p mod 8)+c, so
// eight consecutive lanes each contribute one nibble to a word; three DPP
// OR steps (quad_perm 1032, quad_perm 2301, row_half_mirror) assemble the
// word in every lane of the group of eight and lane 8q stores it.
//
// All arithmetic that feeds a stored fp32 value is one IEEE operation per
// source operation: the file is compiled with contraction off, and division
// and square root are the correctly rounded ones.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#pragma clang fp contract(off)

namespace onebit {

constexpr int kMaxWorkers = 16;

// Hyper-parameters and their fp32-derived constants (computed on the host in
// fp32: a1 = 1-beta1, a2 = 1-beta2, kp = 1+kappa, km = 1-kappa), and the
// variant readings: wd = weight decay lambda (0: off); bias = 1 when the
// warmup direction is bias-corrected by the divisors bc1 = 1-beta1^t and
// bc2 = 1-beta2^t (evaluated in double on the host, rounded once); cd = decay
// of the EMA of the warmup coefficient (0: plain sum) and cd1 = 1-cd.
struct Coef {
  float beta1, beta2, eta, lr, a1, a2, kp, km, c_min, c_max, f_min, f_max;
  float wd, bc1, bc2, cd, cd1;
  int bias;
};

// Warmup direction u = m/(sqrt(v)+eta), or with bias correction
// (m/bc1)/(sqrt(v/bc2)+eta); plus lambda*x with weight decay.
__device__ __forceinline__ float warmup_dir(float m, float v, float x, const Coef& cf) {
  float u = cf.bias ? (m / cf.bc1) / (__builtin_sqrtf(v / cf.bc2) + cf.eta)
                    : m / (__builtin_sqrtf(v) + cf.eta);
  if (cf.wd != 0.0f) u = u + (cf.wd * x);
  return u;
}

// Device view of the tensor table.
struct DevTable {
  const int64_t* off;   // [L+1] flat offset of each tensor
  const int32_t* l0;    // [K] first tensor touched by chunk k
  const int32_t* l1;    // [K] last tensor touched by chunk k
  const int32_t* seg;   // [K] index of segment (k, l0[k]); segment (k, l) = seg[k] + l - l0[k]
  const int32_t* lseg;  // [L+1] segments of tensor l are [lseg[l], lseg[l+1])
  int64_t N;
  int64_t K;
  int32_t L;
};

// Per-worker device pointers, passed by value in the kernel arguments.
struct Workers {
  const float* g[kMaxWorkers];
  float* e[kMaxWorkers];
  uint32_t* bits[kMaxWorkers];
  float* scales[kMaxWorkers];
};

struct PackedIn {
  const uint32_t* bits[kMaxWorkers];
  const float* scales[kMaxWorkers];
};

// Per-worker transmitted values of the sparse stage (entries may be NULL).
struct WorkerVals {
  float* v[kMaxWorkers];
};

// Float4 slots per thread of a chunk's own layout: four from 1024 elements
// up (T = C/16 threads), and below that as many as keep one 64-wide wave per
// chunk: two at 512, one at 256 and below.
template <int C>
constexpr int kSlots = C >= 1024 ? 4 : (C >= 512 ? 2 : 1);

// C elements per chunk, SPT float4 slots per thread, T = G/(4*SPT) threads,
// where G = max(C, 256*SPT) is the workgroup's geometry.  A chunk that
// fills less than one 64-wide wave (SMALL: C < 256*SPT; with its own SPT,
// the chunks of 64 and 128 elements) keeps the geometry of one wave and lies
// in its first C/4 slots: every access is then guarded by the chunk's
// length, as for a partial chunk, and the slots past it are zero.  The
// canonical tree over the padded geometry gives the chunk's own tree bit for
// bit: its extra top levels only add +0 to sums of squares, which are >= +0.
template <int C, int SPT = kSlots<C>>
struct Geo {
  static_assert(C >= 64 && C <= 16384 && (C & (C - 1)) == 0, "chunk must be 2^6..2^14");
  static_assert(SPT == 1 || SPT == 2 || SPT == 4, "slots per thread");
  static constexpr bool SMALL = C < 256 * SPT;
  static constexpr int G = SMALL ? 256 * SPT : C;  // elements a workgroup lays out
  static constexpr int T = G / (4 * SPT);          // threads per chunk
  static constexpr int NW = T / 64;                // waves per chunk
  static constexpr int WORDS = C / 32;             // sign words per chunk
  static_assert(T >= 64 && T <= 1024, "workgroup size");
};

// Whether a chunk takes the guarded path: the partial last chunk (block 0
// of a launch), and every chunk shorter than the workgroup's geometry.
template <int C>
constexpr bool kSmall = Geo<C>::SMALL;

template <int S>
using SlotsN = float[S][4];  // [slot k][component c]
using Slots = SlotsN<4>;
template <int C>
using SlotsOf = SlotsN<kSlots<C>>;  // a chunk's slots in its own layout

// Chunk k of an n-element buffer.  Chunk code is instantiated twice: for the
// full chunks (TAIL = false: nk == C at compile time, no guards) and for the
// one partial last chunk (TAIL = true).  Chunks shorter than the workgroup's
// geometry (Geo::SMALL) take the guarded instantiation for every chunk.
template <int C, bool TAIL>
struct ChunkAt {
  int64_t k, base;
  int nk;
  __device__ __forceinline__ ChunkAt(int64_t k_, int64_t n) {
    k = k_;
    base = k * C;
    // a guarded chunk is the partial last chunk (n - base < C), or any
    // chunk shorter than the geometry
    if constexpr (TAIL && C < 1024) nk = (int)(n - base < C ? n - base : C);
    else nk = TAIL ? (int)(n - base) : C;
  }
};

// ---------------------------------------------------------------------------
// loads and stores of a chunk in the slot layout
// ---------------------------------------------------------------------------
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Streaming (nontemporal) or plain 16-byte accesses, always issued as
// global-memory instructions (the pointers are global; an explicit address
// space keeps the compiler from falling back to flat accesses, which would
// also count against the LDS wait counter at every barrier).
typedef __attribute__((address_space(1))) f32x4 gf32x4;

template <bool NT>
__device__ __forceinline__ f32x4 ld4(const float* p) {
  const gf32x4* q = (const gf32x4*)p;
  if constexpr (NT) return __builtin_nontemporal_load(q);
  else return *q;
}

template <bool NT>
__device__ __forceinline__ void st4(float* p, f32x4 v) {
  gf32x4* q = (gf32x4*)p;
  if constexpr (NT) __builtin_nontemporal_store(v, q);
  else *q = v;
}

template <int C, int SPT = kSlots<C>>
__device__ __forceinline__ bool slot_valid(int k, int c, int nk) {
  return 4 * ((int)threadIdx.x + Geo<C, SPT>::T * k) + c < nk;
}

// A wave-uniform pointer, moved to scalar registers so that loads and stores
// can use a scalar base plus one per-lane 32-bit offset.
template <typename P>
__device__ __forceinline__ P* scalar_ptr(P* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return reinterpret_cast<P*>(((uint64_t)hi << 32) | lo);
}

template <int C, bool TAIL, bool NT = false, int SPT = kSlots<C>>
__device__ __forceinline__ void load_chunk(const float* __restrict__ p, int64_t base, int nk,
                                           SlotsN<SPT>& o) {
  constexpr int T = Geo<C, SPT>::T;
  const int t = threadIdx.x;
  if constexpr (!TAIL) {
#pragma unroll
    for (int k = 0; k < SPT; ++k) {
      // uniform slot base plus one per-lane offset shared by every array
      const char* pk = scalar_ptr(reinterpret_cast<const char*>(p + (base + (int64_t)(4 * T * k))));
      const f32x4 v = ld4<NT>(reinterpret_cast<const float*>(pk + 16u * threadIdx.x));
      o[k][0] = v.x;
      o[k][1] = v.y;
      o[k][2] = v.z;
      o[k][3] = v.w;
    }
  } else if constexpr (C < 1024) {
    // the guarded path of a chunk shorter than 1024 elements (every chunk of
    // 64 or 128 elements, and a partial last chunk): each slot the chunk
    // fills is one 16-byte access (chunks start on a slot boundary, so only
    // a partial last chunk has a slot that is part valid)
#pragma unroll
    for (int k = 0; k < SPT; ++k) {
      const int e0 = 4 * (t + T * k);
      if (e0 + 4 <= nk) {
        const f32x4 v = ld4<NT>(p + (base + e0));
        o[k][0] = v.x;
        o[k][1] = v.y;
        o[k][2] = v.z;
        o[k][3] = v.w;
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) o[k][c] = e0 + c < nk ? p[base + e0 + c] : 0.0f;
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < SPT; ++k)
#pragma unroll
      for (int c = 0; c < 4; ++c) o[k][c] = slot_valid<C, SPT>(k, c, nk) ? p[base + 4 * (t + T * k) + c] : 0.0f;
  }
}

template <int C, bool TAIL, bool NT = false, int SPT = kSlots<C>>
__device__ __forceinline__ void store_chunk(float* __restrict__ p, int64_t base, int nk,
                                            const SlotsN<SPT>& o) {
  constexpr int T = Geo<C, SPT>::T;
  const int t = threadIdx.x;
  if constexpr (!TAIL) {
#pragma unroll
    for (int k = 0; k < SPT; ++k) {
      const f32x4 v = {o[k][0], o[k][1], o[k][2], o[k][3]};
      char* pk = scalar_ptr(reinterpret_cast<char*>(p + (base + (int64_t)(4 * T * k))));
      st4<NT>(reinterpret_cast<float*>(pk + 16u * threadIdx.x), v);
    }
  } else if constexpr (C < 1024) {
#pragma unroll
    for (int k = 0; k < SPT; ++k) {
      const int e0 = 4 * (t + T * k);
      if (e0 + 4 <= nk) {
        st4<NT>(p + (base + e0), f32x4{o[k][0], o[k][1], o[k][2], o[k][3]});
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (e0 + c < nk) p[base + e0 + c] = o[k][c];
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < SPT; ++k)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (slot_valid<C, SPT>(k, c, nk)) p[base + 4 * (t + T * k) + c] = o[k][c];
  }
}

// ---------------------------------------------------------------------------
// canonical chunk sum of squares (see the header comment)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float uniform_f32(float v) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}

// Lanes l < s receive v[l] + v[l+s] for s = 32, 16, 8, 4, 2, 1 in turn, so
// lane 0 ends with the stride-halving tree over the wave's 64 values:
// strides 32 and 16 use the gfx950 lane swaps (the second result of
// permlane32_swap(v, v) holds lane l+32 in lanes 0-31, that of
// permlane16_swap(v, v) lane l+16 in lanes 0-15), strides 8..1 DPP row shifts.
__device__ __forceinline__ float wave_tree_sum(float v) {
  v = v + __uint_as_float(__builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                           false, false)[1]);
  v = v + __uint_as_float(__builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                           false, false)[1]);
  v = v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x108, 0xF, 0xF, false));
  v = v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x104, 0xF, 0xF, false));
  v = v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x102, 0xF, 0xF, false));
  v = v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x101, 0xF, 0xF, false));
  return v;
}

// lds: 2*T float4 (double-buffered between consecutive calls, so one
// barrier per call suffices).  Returns the sum in every thread.  SQ =
// false: z already holds the values to sum (the squares, or partial sums
// of them), and the tree adds them as they are.
template <int C, int SPT = kSlots<C>, bool SQ = true>
__device__ __forceinline__ float chunk_sumsq(const SlotsN<SPT>& z, float4* __restrict__ lds, int& parity) {
  constexpr int T = Geo<C, SPT>::T;
  constexpr int NW = Geo<C, SPT>::NW;
  float p[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    float q[SPT];
#pragma unroll
    for (int k = 0; k < SPT; ++k) q[k] = SQ ? z[k][c] * z[k][c] : z[k][c];
#pragma unroll
    for (int h = SPT / 2; h >= 1; h /= 2)
#pragma unroll
      for (int k = 0; k < h; ++k) q[k] = q[k] + q[k + h];  // slot strides (SPT/2)T .. T
    p[c] = q[0];
  }
  if constexpr (NW > 1) {
    float4* buf = lds + parity * T;
    parity ^= 1;
    buf[threadIdx.x] = make_float4(p[0], p[1], p[2], p[3]);
    __syncthreads();
    const int lane = threadIdx.x & 63;
    float v[NW][4];
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float4 a = buf[w * 64 + lane];
      v[w][0] = a.x;
      v[w][1] = a.y;
      v[w][2] = a.z;
      v[w][3] = a.w;
    }
#pragma unroll
    for (int h = NW / 2; h >= 1; h /= 2)
#pragma unroll
      for (int w = 0; w < h; ++w)
#pragma unroll
        for (int c = 0; c < 4; ++c) v[w][c] = v[w][c] + v[w + h][c];  // thread strides T/2..64
#pragma unroll
    for (int c = 0; c < 4; ++c) p[c] = v[0][c];
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) p[c] = wave_tree_sum(p[c]);  // lane strides 32..1
  return uniform_f32((p[0] + p[2]) + (p[1] + p[3]));  // h = 2, then h = 1
}

__device__ __forceinline__ float chunk_scale(float S, int nk) {
  return __builtin_sqrtf(S) / __builtin_sqrtf((float)nk);
}

// ---------------------------------------------------------------------------
// sign words
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t or_group8(uint32_t x) {
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false);   // quad_perm 1,0,3,2
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, false);   // quad_perm 2,3,0,1
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x141, 0xF, 0xF, false);  // row_half_mirror
  return x;
}

// nib[k]: bit c = sign of element 4(t+T*k)+c.  words: the chunk's C/32 words.
// A chunk shorter than the geometry owns only its first WORDS words; the
// groups of lanes past them neither store nor load.
template <int C, int SPT = kSlots<C>>
__device__ __forceinline__ void store_sign_words(uint32_t* __restrict__ words, const uint32_t (&nib)[SPT]) {
  constexpr int T = Geo<C, SPT>::T;
  const int t = threadIdx.x;
#pragma unroll
  for (int k = 0; k < SPT; ++k) {
    const uint32_t w = or_group8(nib[k] << (4 * (t & 7)));
    const int q = (t + T * k) >> 3;
    if ((t & 7) == 0 && (!Geo<C, SPT>::SMALL || q < Geo<C, SPT>::WORDS)) words[q] = w;
  }
}

template <int C, int SPT = kSlots<C>>
__device__ __forceinline__ void load_sign_nibbles(const uint32_t* __restrict__ words, uint32_t (&nib)[SPT]) {
  constexpr int T = Geo<C, SPT>::T;
  const int t = threadIdx.x;
#pragma unroll
  for (int k = 0; k < SPT; ++k) {
    const int q = (t + T * k) >> 3;
    nib[k] = (!Geo<C, SPT>::SMALL || q < Geo<C, SPT>::WORDS) ? (words[q] >> (4 * (t & 7))) & 0xFu
                                                              : 0u;
  }
}

template <int S>
__device__ __forceinline__ float signed_scale(const uint32_t (&nib)[S], int k, int c, float s) {
  return ((nib[k] >> c) & 1u) ? s : -s;
}

// Error-compensated 1-bit compression of z in place (z becomes the error):
// returns the chunk scale s; nib receives the sign nibbles (0 past the last
// valid element, whose slots are cleared first so they count as 0).
template <int C, bool TAIL, int SPT = kSlots<C>>
__device__ __forceinline__ float compress_slots(SlotsN<SPT>& z, int nk, float4* lds, int& parity,
                                                uint32_t (&nib)[SPT]) {
  if constexpr (TAIL) {
#pragma unroll
    for (int k = 0; k < SPT; ++k)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (!slot_valid<C, SPT>(k, c, nk)) z[k][c] = 0.0f;
  }
  const float s = chunk_scale(chunk_sumsq<C, SPT>(z, lds, parity), nk);
#pragma unroll
  for (int k = 0; k < SPT; ++k) {
    uint32_t nb = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const bool b = z[k][c] >= 0.0f;
      nb |= (uint32_t)(b && (!TAIL || slot_valid<C, SPT>(k, c, nk))) << c;
      z[k][c] = b ? z[k][c] - s : z[k][c] + s;
    }
    nib[k] = nb;
  }
  return s;
}

// ---------------------------------------------------------------------------
// block reductions for per-tensor statistics (fixed order: deterministic)
// ---------------------------------------------------------------------------
// Maximum that propagates NaN: the result is NaN when either operand is,
// else the larger one.  Commutative and associative, so every reduction
// order gives the same value (a rescale ratio that is NaN anywhere in a
// tensor makes its factor NaN, and the status bit reports it).
__device__ __forceinline__ float max_nan(float a, float b) {
  return (a != a) ? a : ((b != b) ? b : fmaxf(a, b));
}

template <int T>
__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) v = max_nan(v, __shfl_xor(v, s, 64));
  if constexpr (T / 64 == 1) {
    return v;
  } else {
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int w = 1; w < T / 64; ++w) r = max_nan(r, red[w]);
    __syncthreads();
    return r;
  }
}

template <int T>
__device__ __forceinline__ void block_sum2(double& a, double& b, double* red) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) {
    a += __shfl_xor(a, s, 64);
    b += __shfl_xor(b, s, 64);
  }
  if constexpr (T / 64 > 1) {
    if ((threadIdx.x & 63) == 0) {
      red[2 * (threadIdx.x >> 6)] = a;
      red[2 * (threadIdx.x >> 6) + 1] = b;
    }
    __syncthreads();
    a = red[0];
    b = red[1];
#pragma unroll
    for (int w = 1; w < T / 64; ++w) {
      a += red[2 * w];
      b += red[2 * w + 1];
    }
    __syncthreads();
  }
}

__device__ __forceinline__ void flag(int32_t* status, int32_t bit) {
  if (status) atomicOr(status, bit);
}

// Tensor of the element at flat index gi within chunk k's tensor range.
__device__ __forceinline__ int tensor_of(const DevTable& tab, int l0, int l1, int64_t gi) {
  int l = l0;
  while (l < l1 && gi >= tab.off[l + 1]) ++l;
  return l;
}

// Per-(chunk, tensor) maximum of q over the chunk's valid elements (NaN if
// any of them is NaN).
template <int C, int SPT = kSlots<C>>
__device__ __forceinline__ void segment_max(const DevTable& tab, int64_t k, int64_t base, int nk,
                                            const SlotsN<SPT>& q, float* red, float* __restrict__ seg_max) {
  constexpr int T = Geo<C, SPT>::T;
  const int l0 = tab.l0[k];
  const int l1 = tab.l1[k];
  const int sb = tab.seg[k];
  for (int l = l0; l <= l1; ++l) {
    const int64_t lo = tab.off[l] - base;
    const int64_t hi = tab.off[l + 1] - base;
    float mx = -__builtin_inff();
#pragma unroll
    for (int a = 0; a < SPT; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int j = 4 * ((int)threadIdx.x + T * a) + c;
        if (j < nk && j >= lo && j < hi) mx = max_nan(mx, q[a][c]);
      }
    mx = block_max<T>(mx, red);
    if (threadIdx.x == 0) seg_max[sb + (l - l0)] = mx;
  }
}

// Per-(chunk, tensor) double sums of a^2 and b^2 over the chunk's valid
// elements (fixed order: per thread, then the wave and block tree).  The two
// sums are reduced independently, so a sum's value does not depend on
// whether the other is formed: HA / HB = false leaves that sum out (its array
// is neither read nor written).  The warmup's two passes both call this, so
// the sum of x^2 that pass 2 carries over for the updated parameters is, bit
// for bit, the one the next step's pass 1 would form from them.
template <int C, int SPT = kSlots<C>, bool HA = true, bool HB = true>
__device__ __forceinline__ void segment_sums(const DevTable& tab, int64_t k, int64_t base, int nk,
                                             const SlotsN<SPT>& a_, const SlotsN<SPT>& b_,
                                             double* red, double* __restrict__ seg_a,
                                             double* __restrict__ seg_b) {
  constexpr int T = Geo<C, SPT>::T;
  const int l0 = tab.l0[k];
  const int l1 = tab.l1[k];
  const int sb = tab.seg[k];
  for (int l = l0; l <= l1; ++l) {
    const int64_t lo = tab.off[l] - base;
    const int64_t hi = tab.off[l + 1] - base;
    double sa = 0.0, sb2 = 0.0;
#pragma unroll
    for (int a = 0; a < SPT; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int j = 4 * ((int)threadIdx.x + T * a) + c;
        if (j < nk && j >= lo && j < hi) {
          if constexpr (HA) sa += (double)a_[a][c] * (double)a_[a][c];
          if constexpr (HB) sb2 += (double)b_[a][c] * (double)b_[a][c];
        }
      }
    block_sum2<T>(sa, sb2, red);
    if (threadIdx.x == 0) {
      if constexpr (HA) seg_a[sb + (l - l0)] = sa;
      if constexpr (HB) seg_b[sb + (l - l0)] = sb2;
    }
  }
}

// ===========================================================================
// kernels
// ===========================================================================

// Launch shape of the element-wise and codec kernels below: one workgroup
// per chunk of an n-element buffer, n_full = n / C full chunks; when the
// buffer ends in a partial chunk, block 0 takes it (its guarded code starts
// first and overlaps the full chunks) and block b > 0 takes full chunk b-1.
// The count is formed with integer division rather than a 64-bit compare,
// which would leave the chunk index in vector registers.
template <int C>
__device__ __forceinline__ int64_t partial_chunks(int64_t n_full, int64_t n) {
  return (n + (C - 1)) / C - n_full;  // 1 if the buffer ends in a partial chunk, else 0
}

// onebit_compress_ef: z = in + err -> bits, scales, err
template <int C, bool TAIL, bool NT>
__device__ __forceinline__ void compress_ef_chunk(int64_t k, int64_t n, const float* __restrict__ in,
                                                  float* __restrict__ err,
                                                  uint32_t* __restrict__ bits,
                                                  float* __restrict__ scales, int32_t* status,
                                                  float4* lds) {
  int parity = 0;
  const ChunkAt<C, TAIL> ch(k, n);
  SlotsOf<C> z, e;
  load_chunk<C, TAIL, NT>(in, ch.base, ch.nk, z);
  load_chunk<C, TAIL, NT>(err, ch.base, ch.nk, e);
#pragma unroll
  for (int a = 0; a < kSlots<C>; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) z[a][c] = z[a][c] + e[a][c];
  uint32_t nib[kSlots<C>];
  const float s = compress_slots<C, TAIL>(z, ch.nk, lds, parity, nib);
  store_chunk<C, TAIL, NT>(err, ch.base, ch.nk, z);
  store_sign_words<C>(bits + ch.k * Geo<C>::WORDS, nib);
  if (threadIdx.x == 0) {
    scales[ch.k] = s;
    if (!__builtin_isfinite(s)) flag(status, 1);
  }
}

template <int C, bool NT = false>
__global__ void __launch_bounds__(Geo<C>::T)
k_compress_ef(int64_t n_full, int64_t n, const float* __restrict__ in, float* __restrict__ err,
              uint32_t* __restrict__ bits, float* __restrict__ scales, int32_t* status) {
  __shared__ float4 lds[2 * Geo<C>::T];
  const int64_t has_tail = partial_chunks<C>(n_full, n);
  if (has_tail && blockIdx.x == 0)
    compress_ef_chunk<C, true, NT>(n_full, n, in, err, bits, scales, status, lds);
  else
    compress_ef_chunk<C, kSmall<C>, NT>((int64_t)blockIdx.x - has_tail, n, in, err, bits, scales,
                                    status, lds);
}

// onebit_average_packed: y = mean of the workers' +-s, + err_s -> recompress
template <int C, bool TAIL, bool NT>
__device__ __forceinline__ void average_packed_chunk(int64_t k, int64_t n, int W, const PackedIn& pin,
                                                     float* __restrict__ err_s,
                                                     uint32_t* __restrict__ bits_out,
                                                     float* __restrict__ scales_out,
                                                     int32_t* status, float4* lds) {
  int parity = 0;
  const ChunkAt<C, TAIL> ch(k, n);
  SlotsOf<C> acc, y;
  for (int w = 0; w < W; ++w) {
    const float s = pin.scales[w][ch.k];
    uint32_t nib[kSlots<C>];
    load_sign_nibbles<C>(pin.bits[w] + ch.k * Geo<C>::WORDS, nib);
#pragma unroll
    for (int a = 0; a < kSlots<C>; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float v = signed_scale(nib, a, c, s);
        acc[a][c] = w == 0 ? v : acc[a][c] + v;
      }
  }
  load_chunk<C, TAIL, NT>(err_s, ch.base, ch.nk, y);
  const float fW = (float)W;
#pragma unroll
  for (int a = 0; a < kSlots<C>; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) y[a][c] = (acc[a][c] / fW) + y[a][c];
  uint32_t nib[kSlots<C>];
  const float s = compress_slots<C, TAIL>(y, ch.nk, lds, parity, nib);
  store_chunk<C, TAIL, NT>(err_s, ch.base, ch.nk, y);
  store_sign_words<C>(bits_out + ch.k * Geo<C>::WORDS, nib);
  if (threadIdx.x == 0) {
    scales_out[ch.k] = s;
    if (!__builtin_isfinite(s)) flag(status, 2);
  }
}

template <int C, bool NT = false>
__global__ void __launch_bounds__(Geo<C>::T)
k_average_packed(int64_t n_full, int64_t n, int W, PackedIn pin, float* __restrict__ err_s,
                 uint32_t* __restrict__ bits_out, float* __restrict__ scales_out, int32_t* status) {
  __shared__ float4 lds[2 * Geo<C>::T];
  const int64_t has_tail = partial_chunks<C>(n_full, n);
  if (has_tail && blockIdx.x == 0)
    average_packed_chunk<C, true, NT>(n_full, n, W, pin, err_s, bits_out, scales_out, status, lds);
  else
    average_packed_chunk<C, kSmall<C>, NT>((int64_t)blockIdx.x - has_tail, n, W, pin, err_s,
                                       bits_out, scales_out, status, lds);
}

// onebit_decompress
template <int C, bool TAIL, bool NT>
__device__ __forceinline__ void decompress_chunk(int64_t k, int64_t n, const uint32_t* __restrict__ bits,
                                                 const float* __restrict__ scales,
                                                 float* __restrict__ out) {
  const ChunkAt<C, TAIL> ch(k, n);
  const float s = scales[ch.k];
  uint32_t nib[kSlots<C>];
  load_sign_nibbles<C>(bits + ch.k * Geo<C>::WORDS, nib);
  SlotsOf<C> o;
#pragma unroll
  for (int a = 0; a < kSlots<C>; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) o[a][c] = signed_scale(nib, a, c, s);
  store_chunk<C, TAIL, NT>(out, ch.base, ch.nk, o);
}

template <int C, bool NT = false>
__global__ void __launch_bounds__(Geo<C>::T)
k_decompress(int64_t n_full, int64_t n, const uint32_t* __restrict__ bits,
             const float* __restrict__ scales, float* __restrict__ out) {
  const int64_t has_tail = partial_chunks<C>(n_full, n);
  if (has_tail && blockIdx.x == 0)
    decompress_chunk<C, true, NT>(n_full, n, bits, scales, out);
  else
    decompress_chunk<C, kSmall<C>, NT>((int64_t)blockIdx.x - has_tail, n, bits, scales, out);
}

// The compressed allreduce of one chunk's momentum: every worker's
// error-compensated 1-bit compression of beta1*m + a1*g_w, then the server's
// average of the W packed chunks and its own error-compensated
// recompression.  On return bm holds beta1*m and nib the server's sign
// nibbles; the server's scale is returned.  With PM (packed momentum) m is
// not read: the momentum is the previous step's server output, which
// bits_s/scales_s hold on entry (chunk k's words and scale are read by this
// workgroup before its first barrier and rewritten after its last one).  With PF, the chunk's slices of
// the two arrays the caller needs next (p0, p1) are loaded into d0, d1 just
// before the server's chunk reduction, so they are in flight across it.
//
// The worker loop carries beta1*m, the running sum ((+-s_0 + +-s_1) + ...)
// of the workers' decompressed values (worker order), and the current
// worker's values.  The kernels built on it are HBM-bound; occupancy (WPE)
// is what moves them.
//   NT:  streaming (nontemporal) loads and stores for the element arrays.
//   PF:  worker w+1's gradient and error are loaded before worker w's chunk
//        reduction, so they are in flight across its barrier.
template <int C, bool TAIL, bool NT, bool PF, int SPT, bool PM>
__device__ __forceinline__ float workers_and_server(const ChunkAt<C, TAIL> ch, int W,
                                                    const Workers& wk, float* __restrict__ err_s,
                                                    const float* __restrict__ m,
                                                    uint32_t* __restrict__ bits_s,
                                                    float* __restrict__ scales_s, const Coef& cf,
                                                    int32_t* status, float4* lds, int& parity,
                                                    SlotsN<SPT>& bm, uint32_t (&nib)[SPT],
                                                    const float* __restrict__ p0,
                                                    const float* __restrict__ p1,
                                                    SlotsN<SPT>& d0, SlotsN<SPT>& d1) {
  const int64_t base = ch.base;
  const int nk = ch.nk;
  const int t = threadIdx.x;

  SlotsN<SPT> acc;
  SlotsN<SPT> gn, en;  // the next worker's gradient and error (PF)
  if constexpr (PF) {
    load_chunk<C, TAIL, NT, SPT>(wk.g[0], base, nk, gn);
    load_chunk<C, TAIL, NT, SPT>(wk.e[0], base, nk, en);
  }
  if constexpr (PM) {
    uint32_t pn[SPT];
    load_sign_nibbles<C, SPT>(bits_s + ch.k * Geo<C>::WORDS, pn);
    const float sp = scales_s[ch.k];
#pragma unroll
    for (int a = 0; a < SPT; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) bm[a][c] = cf.beta1 * signed_scale(pn, a, c, sp);
  } else {
    load_chunk<C, TAIL, NT, SPT>(m, base, nk, bm);
#pragma unroll
    for (int a = 0; a < SPT; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) bm[a][c] = cf.beta1 * bm[a][c];
  }

  for (int w = 0; w < W; ++w) {
    SlotsN<SPT> z, e;
    if constexpr (PF) {
#pragma unroll
      for (int a = 0; a < SPT; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          z[a][c] = gn[a][c];
          e[a][c] = en[a][c];
        }
      if (w + 1 < W) {
        load_chunk<C, TAIL, NT, SPT>(wk.g[w + 1], base, nk, gn);
        load_chunk<C, TAIL, NT, SPT>(wk.e[w + 1], base, nk, en);
      }
    } else {
      load_chunk<C, TAIL, NT, SPT>(wk.g[w], base, nk, z);
      load_chunk<C, TAIL, NT, SPT>(wk.e[w], base, nk, e);
    }
#pragma unroll
    for (int a = 0; a < SPT; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) z[a][c] = (bm[a][c] + (cf.a1 * z[a][c])) + e[a][c];
    uint32_t wnib[SPT];
    const float s = compress_slots<C, TAIL, SPT>(z, nk, lds, parity, wnib);
    store_chunk<C, TAIL, NT, SPT>(wk.e[w], base, nk, z);
    if (wk.bits[w]) store_sign_words<C, SPT>(wk.bits[w] + ch.k * Geo<C>::WORDS, wnib);
#pragma unroll
    for (int a = 0; a < SPT; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float sv = signed_scale(wnib, a, c, s);
        acc[a][c] = w == 0 ? sv : acc[a][c] + sv;
      }
    if (t == 0) {
      if (wk.scales[w]) wk.scales[w][ch.k] = s;
      if (!__builtin_isfinite(s)) flag(status, 1);
    }
  }

  // server: average of the workers' values, add its error, recompress
  SlotsN<SPT> y;
  load_chunk<C, TAIL, NT, SPT>(err_s, base, nk, y);
  const float fW = (float)W;
#pragma unroll
  for (int a = 0; a < SPT; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) y[a][c] = (acc[a][c] / fW) + y[a][c];
  if constexpr (PF) {
    load_chunk<C, TAIL, NT, SPT>(p0, base, nk, d0);
    load_chunk<C, TAIL, NT, SPT>(p1, base, nk, d1);
  }
  const float s2 = compress_slots<C, TAIL, SPT>(y, nk, lds, parity, nib);
  store_chunk<C, TAIL, NT, SPT>(err_s, base, nk, y);
  store_sign_words<C, SPT>(bits_s + ch.k * Geo<C>::WORDS, nib);
  if (t == 0) {
    scales_s[ch.k] = s2;
    if (!__builtin_isfinite(s2)) flag(status, 2);
  }
  return s2;
}

// Pass A after the compressed allreduce, on one chunk: the reconstructed
// gradient from the server's output (nib, s2) and beta1*m (bm), the fresh
// variance (vf in, stored), and the chunk's statistics of the rescale from
// v_frozen (vz): the maximum of the ratio q per (chunk, tensor) segment, or
// (RN, the norm-ratio variant) the double sums of (sqrt(v_frozen)+eta)^2 and
// (sqrt(v_fresh)+eta)^2.
template <int C, bool TAIL, bool NT, int SPT, bool RN>
__device__ __forceinline__ void rescale_chunk(const ChunkAt<C, TAIL>& ch, const DevTable& tab,
                                              const SlotsN<SPT>& bm, const uint32_t (&nib)[SPT],
                                              float s2, SlotsN<SPT>& vf, SlotsN<SPT>& vz,
                                              float* __restrict__ v_fresh,
                                              float* __restrict__ seg_max,
                                              double* __restrict__ seg_z,
                                              double* __restrict__ seg_f, const Coef& cf,
                                              float* red, double* dred) {
#pragma unroll
  for (int a = 0; a < SPT; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float mh = signed_scale(nib, a, c, s2);
      const float gh = (mh - bm[a][c]) / cf.a1;
      vf[a][c] = (cf.beta2 * vf[a][c]) + (cf.a2 * (gh * gh));
    }
  store_chunk<C, TAIL, NT, SPT>(v_fresh, ch.base, ch.nk, vf);
  if constexpr (RN) {
#pragma unroll
    for (int a = 0; a < SPT; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        vz[a][c] = __builtin_sqrtf(vz[a][c]) + cf.eta;
        vf[a][c] = __builtin_sqrtf(vf[a][c]) + cf.eta;
      }
    segment_sums<C, SPT>(tab, ch.k, ch.base, ch.nk, vz, vf, dred, seg_z, seg_f);
  } else {
#pragma unroll
    for (int a = 0; a < SPT; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        vz[a][c] = (__builtin_sqrtf(vz[a][c]) + cf.eta) / (__builtin_sqrtf(vf[a][c]) + cf.eta);
    segment_max<C, SPT>(tab, ch.k, ch.base, ch.nk, vz, red, seg_max);  // vz: the ratio q
  }
}

// 1-bit LAMB compression step, pass A: the compressed allreduce, then the
// reconstructed gradient, the fresh variance and the per-(chunk, tensor)
// statistic of the rescale: the maximum of the ratio q, or (RN, the
// norm-ratio variant) the double sums of (sqrt(v_frozen)+eta)^2 and
// (sqrt(v_fresh)+eta)^2.
template <int C, bool TAIL, bool NT, bool PF, int SPT, bool RN, bool PM>
__device__ __forceinline__ void pass_a_chunk(int64_t kk, const DevTable& tab, int W,
                                             const Workers& wk, float* __restrict__ err_s,
                                             const float* __restrict__ m,
                                             const float* __restrict__ v_frozen,
                                             float* __restrict__ v_fresh,
                                             uint32_t* __restrict__ bits_s,
                                             float* __restrict__ scales_s,
                                             float* __restrict__ seg_max,
                                             double* __restrict__ seg_z,
                                             double* __restrict__ seg_f, const Coef& cf,
                                             int32_t* status, float4* lds, float* red,
                                             double* dred) {
  int parity = 0;
  const ChunkAt<C, TAIL> ch(kk, tab.N);
  const int64_t base = ch.base;
  const int nk = ch.nk;

  SlotsN<SPT> bm, vf, vz;
  uint32_t nib[SPT];
  const float s2 = workers_and_server<C, TAIL, NT, PF, SPT, PM>(ch, W, wk, err_s, m, bits_s,
                                                                scales_s, cf, status, lds, parity,
                                                                bm, nib, v_fresh, v_frozen, vf, vz);

  // reconstructed gradient, fresh variance, rescale ratio
  if constexpr (!PF) {
    load_chunk<C, TAIL, NT, SPT>(v_fresh, base, nk, vf);
    load_chunk<C, TAIL, NT, SPT>(v_frozen, base, nk, vz);
  }
  rescale_chunk<C, TAIL, NT, SPT, RN>(ch, tab, bm, nib, s2, vf, vz, v_fresh, seg_max, seg_z,
                                      seg_f, cf, red, dred);
}


// One workgroup per chunk; when the buffer ends in a partial chunk, block 0
// takes it (its guarded code is slower, so it starts first and overlaps the
// full chunks instead of trailing them).
template <int C, bool NT = false, bool PF = false, int WPE = 1, int SPT = kSlots<C>, bool RN = false,
          bool PM = false>
__global__ void __launch_bounds__((Geo<C, SPT>::T), WPE)
k_compressed_pass_a(int64_t n_full, DevTable tab, int W, Workers wk, float* __restrict__ err_s,
                    const float* __restrict__ m, const float* __restrict__ v_frozen,
                    float* __restrict__ v_fresh, uint32_t* __restrict__ bits_s,
                    float* __restrict__ scales_s, float* __restrict__ seg_max,
                    double* __restrict__ seg_z, double* __restrict__ seg_f, Coef cf,
                    int32_t* status) {
  __shared__ float4 lds[2 * Geo<C, SPT>::T];
  __shared__ float red[Geo<C, SPT>::T / 64];
  __shared__ double dred[RN ? 2 * (Geo<C, SPT>::T / 64) : 1];
  const int64_t has_tail = tab.K - n_full;
  if (has_tail && blockIdx.x == 0)
    pass_a_chunk<C, true, NT, PF, SPT, RN, PM>(n_full, tab, W, wk, err_s, m, v_frozen, v_fresh, bits_s,
                                           scales_s, seg_max, seg_z, seg_f, cf, status, lds, red,
                                           dred);
  else
    pass_a_chunk<C, Geo<C, SPT>::SMALL, NT, PF, SPT, RN, PM>((int64_t)blockIdx.x - has_tail, tab, W, wk, err_s, m,
                                            v_frozen, v_fresh, bits_s, scales_s, seg_max, seg_z,
                                            seg_f, cf, status, lds, red, dred);
}

// 1-bit Adam compression step, first pass: the compressed allreduce of each
// chunk's momentum (every worker, then the server), leaving the server's
// packed output in bits_s/scales_s.  The update x = x - lr*(mhat/(sqrt(
// v_frozen)+eta)), m = mhat follows in k_adam_update, which reads that
// packed output back (C/8 + 4 bytes per chunk).  Interleaved at the
// BERT-Large size, W = 8, the two passes took 7.50 ms against 7.60 ms for
// one pass that also updated x and m (7.02 against 7.15 ms with packed
// momentum), with identical outputs: the single pass held four more
// streams open per chunk.
template <int C, bool TAIL, bool NT, bool PF, int SPT, bool PM>
__device__ __forceinline__ void adam_allreduce_chunk(int64_t kk, int64_t n, int W,
                                                     const Workers& wk, float* __restrict__ err_s,
                                                     const float* __restrict__ m,
                                                     uint32_t* __restrict__ bits_s,
                                                     float* __restrict__ scales_s, const Coef& cf,
                                                     int32_t* status, float4* lds) {
  int parity = 0;
  const ChunkAt<C, TAIL> ch(kk, n);
  SlotsN<SPT> bm, d0, d1;
  uint32_t nib[SPT];
  workers_and_server<C, TAIL, NT, PF, SPT, PM>(ch, W, wk, err_s, m, bits_s, scales_s, cf, status,
                                               lds, parity, bm, nib, nullptr, nullptr, d0, d1);
}

// One worker's part of the compressed allreduce on full chunk k (base =
// k*C) for the persistent pass A: the loop body of workers_and_server.
template <int C, bool NT>
__device__ __forceinline__ void ring_worker(int64_t k, int64_t base, int w, const Workers& wk,
                                            const SlotsOf<C>& bm, SlotsOf<C>& g, const SlotsOf<C>& e, SlotsOf<C>& acc,
                                            const Coef& cf, int32_t* status, float4* lds,
                                            int& parity) {
#pragma unroll
  for (int a = 0; a < kSlots<C>; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) g[a][c] = (bm[a][c] + (cf.a1 * g[a][c])) + e[a][c];
  uint32_t wnib[kSlots<C>];
  const float s = compress_slots<C, false>(g, C, lds, parity, wnib);
  store_chunk<C, false, NT>(wk.e[w], base, C, g);
  if (wk.bits[w]) store_sign_words<C>(wk.bits[w] + k * Geo<C>::WORDS, wnib);
#pragma unroll
  for (int a = 0; a < kSlots<C>; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float sv = signed_scale(wnib, a, c, s);
      acc[a][c] = w == 0 ? sv : acc[a][c] + sv;
    }
  if (threadIdx.x == 0) {
    if (wk.scales[w]) wk.scales[w][k] = s;
    if (!__builtin_isfinite(s)) flag(status, 1);
  }
}

// Pass A as a persistent grid (chunks of up to 4096 elements; the library
// uses it at 4096 with seven or more workers).  A grid of G workgroups,
// sized by the host to one wave per SIMD, steps through the full chunks b,
// b + G, b + 2G, ...; block 0 first takes the partial last chunk through
// pass_a_chunk.  Each workgroup keeps the memory pipe busy across its own
// reductions: while worker w's chunk is reduced, the loads of workers w+1
// and w+2 are in flight (three slot buffers, rotated by unrolling the
// worker loop by three), and across the server's reduction the next
// chunk's momentum and its workers 0-2 are loaded, so no chunk starts
// cold.  Per chunk the arithmetic is pass_a_chunk's, operation for
// operation, so every output is bit for bit the same.  With PM the next
// chunk's momentum is its previous server output (sign words and scale),
// read before this workgroup rewrites them; no other workgroup touches that
// chunk.
template <int C, bool NT, bool RN, bool PM>
__global__ void __launch_bounds__(Geo<C>::T, 1)
k_compressed_pass_a_ring(int64_t n_full, DevTable tab, int W, Workers wk,
                         float* __restrict__ err_s, const float* __restrict__ m,
                         const float* __restrict__ v_frozen, float* __restrict__ v_fresh,
                         uint32_t* __restrict__ bits_s, float* __restrict__ scales_s,
                         float* __restrict__ seg_max, double* __restrict__ seg_z,
                         double* __restrict__ seg_f, Coef cf, int32_t* status) {
  static_assert(!Geo<C>::SMALL && Geo<C>::T <= 256, "one wave per SIMD needs T <= 256");
  constexpr int T = Geo<C>::T;
  __shared__ float4 lds[2 * T];
  __shared__ float red[T / 64];
  __shared__ double dred[RN ? 2 * (T / 64) : 1];
  const int64_t has_tail = tab.K - n_full;
  if (has_tail && blockIdx.x == 0)
    pass_a_chunk<C, true, NT, false, 4, RN, PM>(n_full, tab, W, wk, err_s, m, v_frozen, v_fresh,
                                                bits_s, scales_s, seg_max, seg_z, seg_f, cf,
                                                status, lds, red, dred);
  int64_t k = blockIdx.x;
  if (k >= n_full) return;
  const int64_t G = gridDim.x;
  int parity = 0;

  // the momentum of the chunk ahead: m, or its previous server output
  SlotsOf<C> mn;
  uint32_t pn[kSlots<C>] = {0u, 0u, 0u, 0u};
  float sp = 0.0f;
  // three slot buffers for the workers in flight: worker w in buffer w mod 3
  SlotsOf<C> g0, e0, g1, e1, g2, e2;
  if constexpr (PM) {
    load_sign_nibbles<C>(bits_s + k * Geo<C>::WORDS, pn);
    sp = scales_s[k];
  } else {
    load_chunk<C, false, NT>(m, k * C, C, mn);
  }
  load_chunk<C, false, NT>(wk.g[0], k * C, C, g0);
  load_chunk<C, false, NT>(wk.e[0], k * C, C, e0);
  if (W > 1) {
    load_chunk<C, false, NT>(wk.g[1], k * C, C, g1);
    load_chunk<C, false, NT>(wk.e[1], k * C, C, e1);
  }

  const int t = threadIdx.x;
  const float fW = (float)W;
  for (; k < n_full; k += G) {
    const int64_t base = k * C;
    const int64_t kn = k + G;
    SlotsOf<C> bm, acc;
#pragma unroll
    for (int a = 0; a < kSlots<C>; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if constexpr (PM) bm[a][c] = cf.beta1 * signed_scale(pn, a, c, sp);
        else bm[a][c] = cf.beta1 * mn[a][c];
      }
    if (W > 2 && k == (int64_t)blockIdx.x) {   // later chunks have it in flight already
      load_chunk<C, false, NT>(wk.g[2], base, C, g2);
      load_chunk<C, false, NT>(wk.e[2], base, C, e2);
    }

    for (int w = 0; w < W; w += 3) {
      ring_worker<C, NT>(k, base, w, wk, bm, g0, e0, acc, cf, status, lds, parity);
      if (w + 3 < W) {
        load_chunk<C, false, NT>(wk.g[w + 3], base, C, g0);
        load_chunk<C, false, NT>(wk.e[w + 3], base, C, e0);
      }
      if (w + 1 < W) {
        ring_worker<C, NT>(k, base, w + 1, wk, bm, g1, e1, acc, cf, status, lds, parity);
        if (w + 4 < W) {
          load_chunk<C, false, NT>(wk.g[w + 4], base, C, g1);
          load_chunk<C, false, NT>(wk.e[w + 4], base, C, e1);
        }
      }
      if (w + 2 < W) {
        ring_worker<C, NT>(k, base, w + 2, wk, bm, g2, e2, acc, cf, status, lds, parity);
        if (w + 5 < W) {
          load_chunk<C, false, NT>(wk.g[w + 5], base, C, g2);
          load_chunk<C, false, NT>(wk.e[w + 5], base, C, e2);
        }
      }
    }

    // the server's error, then the next chunk's first loads, then the
    // variances (needed only after the server's reduction)
    SlotsOf<C> y, vf, vz;
    uint32_t nib[kSlots<C>];
    load_chunk<C, false, NT>(err_s, base, C, y);
    if (kn < n_full) {
      if constexpr (PM) {
        load_sign_nibbles<C>(bits_s + kn * Geo<C>::WORDS, pn);
        sp = scales_s[kn];
      } else {
        load_chunk<C, false, NT>(m, kn * C, C, mn);
      }
      load_chunk<C, false, NT>(wk.g[0], kn * C, C, g0);
      load_chunk<C, false, NT>(wk.e[0], kn * C, C, e0);
      if (W > 1) {
        load_chunk<C, false, NT>(wk.g[1], kn * C, C, g1);
        load_chunk<C, false, NT>(wk.e[1], kn * C, C, e1);
      }
      if (W > 2) {
        load_chunk<C, false, NT>(wk.g[2], kn * C, C, g2);
        load_chunk<C, false, NT>(wk.e[2], kn * C, C, e2);
      }
    }
    load_chunk<C, false, NT>(v_fresh, base, C, vf);
    load_chunk<C, false, NT>(v_frozen, base, C, vz);
#pragma unroll
    for (int a = 0; a < kSlots<C>; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) y[a][c] = (acc[a][c] / fW) + y[a][c];
    const float s2 = compress_slots<C, false>(y, C, lds, parity, nib);
    store_chunk<C, false, NT>(err_s, base, C, y);
    store_sign_words<C>(bits_s + k * Geo<C>::WORDS, nib);
    if (t == 0) {
      scales_s[k] = s2;
      if (!__builtin_isfinite(s2)) flag(status, 2);
    }
    const ChunkAt<C, false> ch(k, tab.N);
    rescale_chunk<C, false, NT, 4, RN>(ch, tab, bm, nib, s2, vf, vz, v_fresh, seg_max, seg_z,
                                       seg_f, cf, red, dred);
  }
}

// One workgroup per chunk of an n-element buffer; block 0 takes the partial
// last chunk, if any (as in k_compressed_pass_a).
template <int C, bool NT = false, bool PF = false, int WPE = 1, int SPT = kSlots<C>, bool PM = false>
__global__ void __launch_bounds__((Geo<C, SPT>::T), WPE)
k_adam_allreduce(int64_t n_full, int64_t n, int64_t K, int W, Workers wk,
                 float* __restrict__ err_s, const float* __restrict__ m,
                 uint32_t* __restrict__ bits_s, float* __restrict__ scales_s, Coef cf,
                 int32_t* status) {
  __shared__ float4 lds[2 * Geo<C, SPT>::T];
  const int64_t has_tail = K - n_full;
  if (has_tail && blockIdx.x == 0)
    adam_allreduce_chunk<C, true, NT, PF, SPT, PM>(n_full, n, W, wk, err_s, m, bits_s, scales_s,
                                                   cf, status, lds);
  else
    adam_allreduce_chunk<C, Geo<C, SPT>::SMALL, NT, PF, SPT, PM>((int64_t)blockIdx.x - has_tail, n, W, wk,
                                                    err_s, m, bits_s, scales_s, cf, status, lds);
}

// ---------------------------------------------------------------------------
// One GPU's share of a compression step on W GPUs.  Each GPU compresses its
// own worker's momentum over the whole buffer (k_worker_compress), averages
// and recompresses the chunks it serves, 1/W of them (k_average_packed on
// that range), and, once every GPU holds the server's packed output, forms
// the rescale statistics (k_rescale_stats) and updates its replica
// (k_rescale_finalize, k_compressed_pass_b).  The arithmetic is that of the
// fused k_compressed_pass_a, element for element, so both give the same
// bits.
// ---------------------------------------------------------------------------

// beta1*m for one chunk: from the fp32 momentum or (PM) from the previous
// server output (bits_m, scales_m), whose decompressed value is the momentum.
template <int C, bool TAIL, bool NT, bool PM>
__device__ __forceinline__ void beta1_momentum(const ChunkAt<C, TAIL>& ch,
                                               const float* __restrict__ m,
                                               const uint32_t* __restrict__ bits_m,
                                               const float* __restrict__ scales_m, const Coef& cf,
                                               SlotsOf<C>& bm) {
  if constexpr (PM) {
    uint32_t pn[kSlots<C>];
    load_sign_nibbles<C>(bits_m + ch.k * Geo<C>::WORDS, pn);
    const float sp = scales_m[ch.k];
#pragma unroll
    for (int a = 0; a < kSlots<C>; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) bm[a][c] = cf.beta1 * signed_scale(pn, a, c, sp);
  } else {
    load_chunk<C, TAIL, NT>(m, ch.base, ch.nk, bm);
#pragma unroll
    for (int a = 0; a < kSlots<C>; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) bm[a][c] = cf.beta1 * bm[a][c];
  }
}

// One worker: z = (beta1*m + a1*g) + e, error-compensated 1-bit compression.
template <int C, bool TAIL, bool NT, bool PM>
__device__ __forceinline__ void worker_compress_chunk(int64_t k, int64_t n, const float* __restrict__ g,
                                                      float* __restrict__ e,
                                                      const float* __restrict__ m,
                                                      const uint32_t* __restrict__ bits_m,
                                                      const float* __restrict__ scales_m,
                                                      uint32_t* __restrict__ bits_w,
                                                      float* __restrict__ scales_w, const Coef& cf,
                                                      int32_t* status, float4* lds) {
  int parity = 0;
  const ChunkAt<C, TAIL> ch(k, n);
  SlotsOf<C> z, gg, ee;
  beta1_momentum<C, TAIL, NT, PM>(ch, m, bits_m, scales_m, cf, z);
  load_chunk<C, TAIL, NT>(g, ch.base, ch.nk, gg);
  load_chunk<C, TAIL, NT>(e, ch.base, ch.nk, ee);
#pragma unroll
  for (int a = 0; a < kSlots<C>; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) z[a][c] = (z[a][c] + (cf.a1 * gg[a][c])) + ee[a][c];
  uint32_t nib[kSlots<C>];
  const float s = compress_slots<C, TAIL>(z, ch.nk, lds, parity, nib);
  store_chunk<C, TAIL, NT>(e, ch.base, ch.nk, z);
  store_sign_words<C>(bits_w + ch.k * Geo<C>::WORDS, nib);
  if (threadIdx.x == 0) {
    scales_w[ch.k] = s;
    if (!__builtin_isfinite(s)) flag(status, 1);
  }
}

template <int C, bool NT = true, bool PM = false>
__global__ void __launch_bounds__(Geo<C>::T)
k_worker_compress(int64_t n_full, int64_t n, const float* __restrict__ g, float* __restrict__ e,
                  const float* __restrict__ m, const uint32_t* __restrict__ bits_m,
                  const float* __restrict__ scales_m, uint32_t* __restrict__ bits_w,
                  float* __restrict__ scales_w, Coef cf, int32_t* status) {
  __shared__ float4 lds[2 * Geo<C>::T];
  const int64_t has_tail = partial_chunks<C>(n_full, n);
  if (has_tail && blockIdx.x == 0)
    worker_compress_chunk<C, true, NT, PM>(n_full, n, g, e, m, bits_m, scales_m, bits_w, scales_w,
                                           cf, status, lds);
  else
    worker_compress_chunk<C, kSmall<C>, NT, PM>((int64_t)blockIdx.x - has_tail, n, g, e, m, bits_m,
                                            scales_m, bits_w, scales_w, cf, status, lds);
}

// The receiver side of the rescale: mhat from the server's packed output,
// the reconstructed gradient, the fresh variance, and the per-(chunk,
// tensor) statistic of the rescale (as the second half of pass A).
template <int C, bool TAIL, bool NT, bool RN, bool PM>
__device__ __forceinline__ void rescale_stats_chunk(int64_t kk, const DevTable& tab,
                                                    const uint32_t* __restrict__ bits_s,
                                                    const float* __restrict__ scales_s,
                                                    const float* __restrict__ m,
                                                    const uint32_t* __restrict__ bits_m,
                                                    const float* __restrict__ scales_m,
                                                    const float* __restrict__ v_frozen,
                                                    float* __restrict__ v_fresh,
                                                    float* __restrict__ seg_max,
                                                    double* __restrict__ seg_z,
                                                    double* __restrict__ seg_f, const Coef& cf,
                                                    float* red, double* dred) {
  const ChunkAt<C, TAIL> ch(kk, tab.N);
  const int64_t base = ch.base;
  const int nk = ch.nk;
  uint32_t nib[kSlots<C>];
  load_sign_nibbles<C>(bits_s + ch.k * Geo<C>::WORDS, nib);
  const float s2 = scales_s[ch.k];
  SlotsOf<C> bm, vf, vz;
  beta1_momentum<C, TAIL, NT, PM>(ch, m, bits_m, scales_m, cf, bm);
  load_chunk<C, TAIL, NT>(v_fresh, base, nk, vf);
  load_chunk<C, TAIL, NT>(v_frozen, base, nk, vz);
#pragma unroll
  for (int a = 0; a < kSlots<C>; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float mh = signed_scale(nib, a, c, s2);
      const float gh = (mh - bm[a][c]) / cf.a1;
      vf[a][c] = (cf.beta2 * vf[a][c]) + (cf.a2 * (gh * gh));
    }
  store_chunk<C, TAIL, NT>(v_fresh, base, nk, vf);
  if constexpr (RN) {
#pragma unroll
    for (int a = 0; a < kSlots<C>; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        vz[a][c] = __builtin_sqrtf(vz[a][c]) + cf.eta;
        vf[a][c] = __builtin_sqrtf(vf[a][c]) + cf.eta;
      }
    segment_sums<C>(tab, ch.k, base, nk, vz, vf, dred, seg_z, seg_f);
  } else {
#pragma unroll
    for (int a = 0; a < kSlots<C>; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        vz[a][c] = (__builtin_sqrtf(vz[a][c]) + cf.eta) / (__builtin_sqrtf(vf[a][c]) + cf.eta);
    segment_max<C>(tab, ch.k, base, nk, vz, red, seg_max);
  }
}

template <int C, bool NT = true, bool RN = false, bool PM = false>
__global__ void __launch_bounds__(Geo<C>::T)
k_rescale_stats(int64_t n_full, DevTable tab, const uint32_t* __restrict__ bits_s,
                const float* __restrict__ scales_s, const float* __restrict__ m,
                const uint32_t* __restrict__ bits_m, const float* __restrict__ scales_m,
                const float* __restrict__ v_frozen, float* __restrict__ v_fresh,
                float* __restrict__ seg_max, double* __restrict__ seg_z,
                double* __restrict__ seg_f, Coef cf) {
  __shared__ float red[Geo<C>::T / 64];
  __shared__ double dred[RN ? 2 * (Geo<C>::T / 64) : 1];
  const int64_t has_tail = tab.K - n_full;
  if (has_tail && blockIdx.x == 0)
    rescale_stats_chunk<C, true, NT, RN, PM>(n_full, tab, bits_s, scales_s, m, bits_m, scales_m,
                                             v_frozen, v_fresh, seg_max, seg_z, seg_f, cf, red,
                                             dred);
  else
    rescale_stats_chunk<C, kSmall<C>, NT, RN, PM>((int64_t)blockIdx.x - has_tail, tab, bits_s,
                                              scales_s, m, bits_m, scales_m, v_frozen, v_fresh,
                                              seg_max, seg_z, seg_f, cf, red, dred);
}

// 1-bit Adam on a receiver: x = x - lr*(mhat/(sqrt(v_frozen)+eta)) and
// m = mhat (m NULL: packed momentum), mhat from the server's packed output
// (the second pass of the 1-bit Adam step, after k_adam_allreduce).
template <int C, bool TAIL, bool NT>
__device__ __forceinline__ void adam_update_chunk(int64_t k, int64_t n,
                                                  const uint32_t* __restrict__ bits_s,
                                                  const float* __restrict__ scales_s,
                                                  const float* __restrict__ v_frozen,
                                                  float* __restrict__ x, float* __restrict__ m,
                                                  const Coef& cf) {
  const ChunkAt<C, TAIL> ch(k, n);
  uint32_t nib[kSlots<C>];
  load_sign_nibbles<C>(bits_s + ch.k * Geo<C>::WORDS, nib);
  const float s2 = scales_s[ch.k];
  SlotsOf<C> xx, vz, mh;
  load_chunk<C, TAIL, NT>(x, ch.base, ch.nk, xx);
  load_chunk<C, TAIL, NT>(v_frozen, ch.base, ch.nk, vz);
#pragma unroll
  for (int a = 0; a < kSlots<C>; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      mh[a][c] = signed_scale(nib, a, c, s2);
      xx[a][c] = xx[a][c] - (cf.lr * (mh[a][c] / (__builtin_sqrtf(vz[a][c]) + cf.eta)));
    }
  store_chunk<C, TAIL, NT>(x, ch.base, ch.nk, xx);
  if (m) store_chunk<C, TAIL, NT>(m, ch.base, ch.nk, mh);
}

template <int C, bool NT = true>
__global__ void __launch_bounds__(Geo<C>::T)
k_adam_update(int64_t n_full, int64_t n, const uint32_t* __restrict__ bits_s,
              const float* __restrict__ scales_s, const float* __restrict__ v_frozen,
              float* __restrict__ x, float* __restrict__ m, Coef cf) {
  const int64_t has_tail = partial_chunks<C>(n_full, n);
  if (has_tail && blockIdx.x == 0)
    adam_update_chunk<C, true, NT>(n_full, n, bits_s, scales_s, v_frozen, x, m, cf);
  else
    adam_update_chunk<C, kSmall<C>, NT>((int64_t)blockIdx.x - has_tail, n, bits_s, scales_s, v_frozen,
                                    x, m, cf);
}

// 1-bit Adam warmup: one Adam step, element-wise in one pass (mean gradient,
// moments, x = x - lr*(m/(sqrt(v)+eta))).
template <int C, bool TAIL, int SPT, int DEPTH>
__device__ __forceinline__ void adam_warmup_chunk(int64_t k, int64_t n, int W, const Workers& wk,
                                                  float* __restrict__ x, float* __restrict__ m,
                                                  float* __restrict__ v, const Coef& cf) {
  const ChunkAt<C, TAIL> ch(k, n);
  const int64_t base = ch.base;
  const int nk = ch.nk;
  // gradients summed in worker order with DEPTH of them in flight, as in the
  // LAMB warmup's first pass; m, v and x loaded once the last gradient has
  // been asked for
  SlotsN<SPT> gs, mm, vv, xx;
  SlotsN<SPT> q[DEPTH];
  load_chunk<C, TAIL, true, SPT>(wk.g[0], base, nk, gs);
#pragma unroll
  for (int d = 0; d < DEPTH; ++d)
    if (1 + d < W) load_chunk<C, TAIL, true, SPT>(wk.g[1 + d], base, nk, q[d]);
  if (W <= DEPTH) {
    load_chunk<C, TAIL, true, SPT>(m, base, nk, mm);
    load_chunk<C, TAIL, true, SPT>(v, base, nk, vv);
    load_chunk<C, TAIL, true, SPT>(x, base, nk, xx);
  }
  for (int w = 1; w < W; ++w) {
    SlotsN<SPT> g;
#pragma unroll
    for (int a = 0; a < SPT; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) g[a][c] = q[0][a][c];
#pragma unroll
    for (int d = 0; d + 1 < DEPTH; ++d)
#pragma unroll
      for (int a = 0; a < SPT; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c) q[d][a][c] = q[d + 1][a][c];
    if (w + DEPTH < W) {
      load_chunk<C, TAIL, true, SPT>(wk.g[w + DEPTH], base, nk, q[DEPTH - 1]);
    } else if (w + DEPTH == W) {
      load_chunk<C, TAIL, true, SPT>(m, base, nk, mm);
      load_chunk<C, TAIL, true, SPT>(v, base, nk, vv);
      load_chunk<C, TAIL, true, SPT>(x, base, nk, xx);
    }
#pragma unroll
    for (int a = 0; a < SPT; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) gs[a][c] = gs[a][c] + g[a][c];
  }
  const float fW = (float)W;
#pragma unroll
  for (int a = 0; a < SPT; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float gb = gs[a][c] / fW;
      mm[a][c] = (cf.beta1 * mm[a][c]) + (cf.a1 * gb);
      vv[a][c] = (cf.beta2 * vv[a][c]) + (cf.a2 * (gb * gb));
      const float u = warmup_dir(mm[a][c], vv[a][c], xx[a][c], cf);
      xx[a][c] = xx[a][c] - (cf.lr * u);
    }
  store_chunk<C, TAIL, true, SPT>(m, base, nk, mm);
  store_chunk<C, TAIL, true, SPT>(v, base, nk, vv);
  store_chunk<C, TAIL, true, SPT>(x, base, nk, xx);
}

template <int C, int WPE = 1, int SPT = kSlots<C>, int DEPTH = 1>
__global__ void __launch_bounds__((Geo<C, SPT>::T), WPE)
k_adam_warmup(int64_t n_full, int64_t n, int W, Workers wk, float* __restrict__ x,
              float* __restrict__ m, float* __restrict__ v, Coef cf) {
  const int64_t has_tail = partial_chunks<C>(n_full, n);
  if (has_tail && blockIdx.x == 0)
    adam_warmup_chunk<C, true, SPT, DEPTH>(n_full, n, W, wk, x, m, v, cf);
  else
    adam_warmup_chunk<C, Geo<C, SPT>::SMALL, SPT, DEPTH>((int64_t)blockIdx.x - has_tail, n, W, wk, x, m, v,
                                                cf);
}

// SLAMB-style sparse compression stage, one pass per chunk.  The chunk's
// C/64 blocks of 64 elements are transmitted in nsel consecutive blocks from
// block sel[k] (cyclically); thread t's slot k covers block (t + T*k)/16, so
// 16 consecutive lanes share one block and its selection.  Workers' values
// are error-compensated on the unselected blocks and averaged on the
// selected ones; the momentum is masked to the selected blocks, where the
// fresh variance, the clamped element-wise ratio and the update follow.
template <int C, bool TAIL, bool NT>
__device__ __forceinline__ void sparse_chunk(int64_t kk, const DevTable& tab, int W, int nsel,
                                             const int32_t* __restrict__ sel, const Workers& wk,
                                             const WorkerVals& vals_w, float* __restrict__ x,
                                             float* __restrict__ m,
                                             const float* __restrict__ v_frozen,
                                             float* __restrict__ v_fresh,
                                             const float* __restrict__ c_avg,
                                             float* __restrict__ vals_s, const Coef& cf,
                                             int32_t* status) {
  constexpr int T = Geo<C>::T;
  constexpr int NB = C / 64;
  const ChunkAt<C, TAIL> ch(kk, tab.N);
  const int64_t base = ch.base;
  const int nk = ch.nk;
  const int t = threadIdx.x;
  const int b0 = ((sel[ch.k] % NB) + NB) % NB;
  const int64_t per = (int64_t)nsel * 64;
  // per slot: transmitted position within the chunk's values, or -1
  int pos[kSlots<C>];
#pragma unroll
  for (int a = 0; a < kSlots<C>; ++a) {
    const int p = t + T * a;                    // float4 slot; block p/16
    const int rel = ((p / 16) - b0 + NB) % NB;
    pos[a] = ((!Geo<C>::SMALL || p < C / 4) && rel < nsel) ? rel * 64 + 4 * (p % 16) : -1;
  }

  SlotsOf<C> bm, acc;
  load_chunk<C, TAIL, NT>(m, base, nk, bm);
#pragma unroll
  for (int a = 0; a < kSlots<C>; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) bm[a][c] = cf.beta1 * bm[a][c];

  for (int w = 0; w < W; ++w) {
    SlotsOf<C> z, e;
    load_chunk<C, TAIL, NT>(wk.g[w], base, nk, z);
    load_chunk<C, TAIL, NT>(wk.e[w], base, nk, e);
    float* vw = vals_w.v[w];
#pragma unroll
    for (int a = 0; a < kSlots<C>; ++a) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        z[a][c] = (bm[a][c] + (cf.a1 * z[a][c])) + e[a][c];
        if (pos[a] >= 0) {
          acc[a][c] = w == 0 ? z[a][c] : acc[a][c] + z[a][c];
          e[a][c] = 0.0f;
        } else {
          e[a][c] = z[a][c];
        }
      }
      if (vw && pos[a] >= 0) {
        float* q = vw + ch.k * per + pos[a];
        if constexpr (TAIL) {
#pragma unroll
          for (int c = 0; c < 4; ++c) q[c] = slot_valid<C>(a, c, nk) ? z[a][c] : 0.0f;
        } else {
          st4<NT>(q, f32x4{z[a][0], z[a][1], z[a][2], z[a][3]});
        }
      }
    }
    store_chunk<C, TAIL, NT>(wk.e[w], base, nk, e);
  }

  // server average, masked momentum
  const float fW = (float)W;
#pragma unroll
  for (int a = 0; a < kSlots<C>; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[a][c] = pos[a] >= 0 ? acc[a][c] / fW : 0.0f;

  // element-wise rescale and update on the transmitted blocks
  const int l0 = tab.l0[ch.k];
  const int l1 = tab.l1[ch.k];
  const float st0 = cf.lr * c_avg[l0];
#pragma unroll
  for (int a = 0; a < kSlots<C>; ++a) {
    if (pos[a] < 0) continue;
    const int64_t e0 = base + 4 * (t + T * a);
    float xs[4], vz[4], vf[4];
    if constexpr (TAIL) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bool ok = slot_valid<C>(a, c, nk);
        xs[c] = ok ? x[e0 + c] : 0.0f;
        vz[c] = ok ? v_frozen[e0 + c] : 0.0f;
        vf[c] = ok ? v_fresh[e0 + c] : 0.0f;
      }
    } else {
      const f32x4 xv = ld4<NT>(x + e0), zv = ld4<NT>(v_frozen + e0), fv = ld4<NT>(v_fresh + e0);
      xs[0] = xv.x; xs[1] = xv.y; xs[2] = xv.z; xs[3] = xv.w;
      vz[0] = zv.x; vz[1] = zv.y; vz[2] = zv.z; vz[3] = zv.w;
      vf[0] = fv.x; vf[1] = fv.y; vf[2] = fv.z; vf[3] = fv.w;
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float mh = acc[a][c];
      const float gh = (mh - bm[a][c]) / cf.a1;
      vf[c] = (cf.beta2 * vf[c]) + (cf.a2 * (gh * gh));
      const float dz = __builtin_sqrtf(vz[c]) + cf.eta;
      const float q = dz / (__builtin_sqrtf(vf[c]) + cf.eta);
      const float r = fminf(fmaxf(q, cf.f_min), cf.f_max);
      const float stp = l0 == l1 ? st0 : cf.lr * c_avg[tensor_of(tab, l0, l1, e0 + c)];
      xs[c] = xs[c] - (stp * (r * (mh / dz)));
      if (!__builtin_isfinite(mh)) flag(status, 2);
    }
    float* q = vals_s + ch.k * per + pos[a];
    if constexpr (TAIL) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (slot_valid<C>(a, c, nk)) {
          x[e0 + c] = xs[c];
          v_fresh[e0 + c] = vf[c];
        }
        q[c] = slot_valid<C>(a, c, nk) ? acc[a][c] : 0.0f;
      }
    } else {
      st4<NT>(x + e0, f32x4{xs[0], xs[1], xs[2], xs[3]});
      st4<NT>(v_fresh + e0, f32x4{vf[0], vf[1], vf[2], vf[3]});
      st4<NT>(q, f32x4{acc[a][0], acc[a][1], acc[a][2], acc[a][3]});
    }
  }
  store_chunk<C, TAIL, NT>(m, base, nk, acc);
}

// ---------------------------------------------------------------------------
// One GPU's share of a W-GPU sparse step: its worker's transmitted values
// and local error (k_sparse_worker), the mean of the W workers' values on the
// chunks it serves (k_mean_values), and, with every chunk's mean in hand,
// the masked momentum, fresh variance and update of its replica
// (k_sparse_update).  Same arithmetic as sparse_chunk, element for element.
// ---------------------------------------------------------------------------

// Transmitted position of thread t's slots within the chunk's values, or -1.
template <int C>
__device__ __forceinline__ void sparse_positions(int32_t sel_k, int nsel, int (&pos)[kSlots<C>]) {
  constexpr int T = Geo<C>::T;
  constexpr int NB = C / 64;
  const int b0 = ((sel_k % NB) + NB) % NB;
#pragma unroll
  for (int a = 0; a < kSlots<C>; ++a) {
    const int p = (int)threadIdx.x + T * a;
    const int rel = ((p / 16) - b0 + NB) % NB;
    pos[a] = ((!Geo<C>::SMALL || p < C / 4) && rel < nsel) ? rel * 64 + 4 * (p % 16) : -1;
  }
}

template <int C, bool TAIL, bool NT>
__device__ __forceinline__ void sparse_worker_chunk(int64_t k, int64_t n, int nsel,
                                                    const int32_t* __restrict__ sel,
                                                    const float* __restrict__ g,
                                                    float* __restrict__ e,
                                                    const float* __restrict__ m,
                                                    float* __restrict__ vals, const Coef& cf) {
  const ChunkAt<C, TAIL> ch(k, n);
  const int64_t per = (int64_t)nsel * 64;
  int pos[kSlots<C>];
  sparse_positions<C>(sel[ch.k], nsel, pos);
  SlotsOf<C> z, gg, ee;
  load_chunk<C, TAIL, NT>(m, ch.base, ch.nk, z);
  load_chunk<C, TAIL, NT>(g, ch.base, ch.nk, gg);
  load_chunk<C, TAIL, NT>(e, ch.base, ch.nk, ee);
#pragma unroll
  for (int a = 0; a < kSlots<C>; ++a) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      z[a][c] = ((cf.beta1 * z[a][c]) + (cf.a1 * gg[a][c])) + ee[a][c];
      ee[a][c] = pos[a] >= 0 ? 0.0f : z[a][c];
    }
    if (pos[a] >= 0) {
      float* q = vals + ch.k * per + pos[a];
      if constexpr (TAIL) {
#pragma unroll
        for (int c = 0; c < 4; ++c) q[c] = slot_valid<C>(a, c, ch.nk) ? z[a][c] : 0.0f;
      } else {
        st4<NT>(q, f32x4{z[a][0], z[a][1], z[a][2], z[a][3]});
      }
    }
  }
  store_chunk<C, TAIL, NT>(e, ch.base, ch.nk, ee);
}

template <int C, bool NT = true>
__global__ void __launch_bounds__(Geo<C>::T)
k_sparse_worker(int64_t n_full, int64_t n, int nsel, const int32_t* __restrict__ sel,
                const float* __restrict__ g, float* __restrict__ e, const float* __restrict__ m,
                float* __restrict__ vals, Coef cf) {
  const int64_t has_tail = partial_chunks<C>(n_full, n);
  if (has_tail && blockIdx.x == 0)
    sparse_worker_chunk<C, true, NT>(n_full, n, nsel, sel, g, e, m, vals, cf);
  else
    sparse_worker_chunk<C, kSmall<C>, NT>((int64_t)blockIdx.x - has_tail, n, nsel, sel, g, e, m, vals,
                                      cf);
}

// out[i] = ((v_0[i] + v_1[i]) + ...) / W over count4 float4 groups.
template <bool NT = true>
__global__ void __launch_bounds__(256)
k_mean_values(int64_t count4, int W, WorkerVals vals_w, float* __restrict__ out) {
  const float fW = (float)W;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < count4;
       i += (int64_t)gridDim.x * 256) {
    f32x4 acc = ld4<NT>(vals_w.v[0] + 4 * i);
    for (int w = 1; w < W; ++w) {
      const f32x4 v = ld4<NT>(vals_w.v[w] + 4 * i);
      acc.x = acc.x + v.x;
      acc.y = acc.y + v.y;
      acc.z = acc.z + v.z;
      acc.w = acc.w + v.w;
    }
    st4<NT>(out + 4 * i, f32x4{acc.x / fW, acc.y / fW, acc.z / fW, acc.w / fW});
  }
}

template <int C, bool TAIL, bool NT>
__device__ __forceinline__ void sparse_update_chunk(int64_t kk, const DevTable& tab, int nsel,
                                                    const int32_t* __restrict__ sel,
                                                    const float* __restrict__ vals_s,
                                                    float* __restrict__ x, float* __restrict__ m,
                                                    const float* __restrict__ v_frozen,
                                                    float* __restrict__ v_fresh,
                                                    const float* __restrict__ c_avg,
                                                    const Coef& cf, int32_t* status) {
  constexpr int T = Geo<C>::T;
  const ChunkAt<C, TAIL> ch(kk, tab.N);
  const int64_t base = ch.base;
  const int nk = ch.nk;
  const int t = threadIdx.x;
  const int64_t per = (int64_t)nsel * 64;
  int pos[kSlots<C>];
  sparse_positions<C>(sel[ch.k], nsel, pos);
  // mhat: the server's mean on the selection, 0 elsewhere.  The previous
  // momentum enters only through ghat on the selection, so m is read there
  // alone (elsewhere it is overwritten with 0 unread).
  SlotsOf<C> bm, mh;
#pragma unroll
  for (int a = 0; a < kSlots<C>; ++a) {
    if (pos[a] >= 0) {
      const f32x4 v = ld4<NT>(vals_s + ch.k * per + pos[a]);
      mh[a][0] = v.x; mh[a][1] = v.y; mh[a][2] = v.z; mh[a][3] = v.w;
      const int64_t e0 = base + 4 * (t + T * a);
      if constexpr (TAIL) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
          bm[a][c] = cf.beta1 * (slot_valid<C>(a, c, nk) ? m[e0 + c] : 0.0f);
      } else {
        const f32x4 mv = ld4<NT>(m + e0);
        bm[a][0] = cf.beta1 * mv.x; bm[a][1] = cf.beta1 * mv.y;
        bm[a][2] = cf.beta1 * mv.z; bm[a][3] = cf.beta1 * mv.w;
      }
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) mh[a][c] = bm[a][c] = 0.0f;
    }
  }
  const int l0 = tab.l0[ch.k];
  const int l1 = tab.l1[ch.k];
  const float st0 = cf.lr * c_avg[l0];
#pragma unroll
  for (int a = 0; a < kSlots<C>; ++a) {
    if (pos[a] < 0) continue;
    const int64_t e0 = base + 4 * (t + T * a);
    float xs[4], vz[4], vf[4];
    if constexpr (TAIL) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bool ok = slot_valid<C>(a, c, nk);
        xs[c] = ok ? x[e0 + c] : 0.0f;
        vz[c] = ok ? v_frozen[e0 + c] : 0.0f;
        vf[c] = ok ? v_fresh[e0 + c] : 0.0f;
      }
    } else {
      const f32x4 xv = ld4<NT>(x + e0), zv = ld4<NT>(v_frozen + e0), fv = ld4<NT>(v_fresh + e0);
      xs[0] = xv.x; xs[1] = xv.y; xs[2] = xv.z; xs[3] = xv.w;
      vz[0] = zv.x; vz[1] = zv.y; vz[2] = zv.z; vz[3] = zv.w;
      vf[0] = fv.x; vf[1] = fv.y; vf[2] = fv.z; vf[3] = fv.w;
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float gh = (mh[a][c] - bm[a][c]) / cf.a1;
      vf[c] = (cf.beta2 * vf[c]) + (cf.a2 * (gh * gh));
      const float dz = __builtin_sqrtf(vz[c]) + cf.eta;
      const float q = dz / (__builtin_sqrtf(vf[c]) + cf.eta);
      const float r = fminf(fmaxf(q, cf.f_min), cf.f_max);
      const float stp = l0 == l1 ? st0 : cf.lr * c_avg[tensor_of(tab, l0, l1, e0 + c)];
      xs[c] = xs[c] - (stp * (r * (mh[a][c] / dz)));
      if (!__builtin_isfinite(mh[a][c])) flag(status, 2);
    }
    if constexpr (TAIL) {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (slot_valid<C>(a, c, nk)) {
          x[e0 + c] = xs[c];
          v_fresh[e0 + c] = vf[c];
        }
    } else {
      st4<NT>(x + e0, f32x4{xs[0], xs[1], xs[2], xs[3]});
      st4<NT>(v_fresh + e0, f32x4{vf[0], vf[1], vf[2], vf[3]});
    }
  }
  store_chunk<C, TAIL, NT>(m, base, nk, mh);
}

template <int C, bool NT = true>
__global__ void __launch_bounds__(Geo<C>::T)
k_sparse_update(int64_t n_full, DevTable tab, int nsel, const int32_t* __restrict__ sel,
                const float* __restrict__ vals_s, float* __restrict__ x, float* __restrict__ m,
                const float* __restrict__ v_frozen, float* __restrict__ v_fresh,
                const float* __restrict__ c_avg, Coef cf, int32_t* status) {
  const int64_t has_tail = tab.K - n_full;
  if (has_tail && blockIdx.x == 0)
    sparse_update_chunk<C, true, NT>(n_full, tab, nsel, sel, vals_s, x, m, v_frozen, v_fresh,
                                     c_avg, cf, status);
  else
    sparse_update_chunk<C, kSmall<C>, NT>((int64_t)blockIdx.x - has_tail, tab, nsel, sel, vals_s, x, m,
                                      v_frozen, v_fresh, c_avg, cf, status);
}

// One workgroup per chunk; block 0 takes the partial last chunk, if any.
template <int C, bool NT = true, int WPE = 1>
__global__ void __launch_bounds__(Geo<C>::T, WPE)
k_sparse_step(int64_t n_full, DevTable tab, int W, int nsel, const int32_t* __restrict__ sel,
              Workers wk, WorkerVals vals_w, float* __restrict__ x, float* __restrict__ m,
              const float* __restrict__ v_frozen, float* __restrict__ v_fresh,
              const float* __restrict__ c_avg, float* __restrict__ vals_s, Coef cf,
              int32_t* status) {
  const int64_t has_tail = tab.K - n_full;
  if (has_tail && blockIdx.x == 0)
    sparse_chunk<C, true, NT>(n_full, tab, W, nsel, sel, wk, vals_w, x, m, v_frozen, v_fresh,
                              c_avg, vals_s, cf, status);
  else
    sparse_chunk<C, kSmall<C>, NT>((int64_t)blockIdx.x - has_tail, tab, W, nsel, sel, wk, vals_w, x, m,
                               v_frozen, v_fresh, c_avg, vals_s, cf, status);
}

// A thread's share of a tensor's reduction over its segments [lo, hi):
// segments lo + t, lo + t + TB, ...  With U = 1 one running value; with
// U > 1 (a tensor of many segments) the segments are taken in rounds of
// U*TB, each round's U loads per thread issued together (predicated past
// hi) into U running values, which are then combined pairwise.  The order
// is fixed by (TB, U) and the segment range, so the result is
// reproducible; the maximum does not depend on it.
template <int TB, int U>
__device__ __forceinline__ float thread_seg_max(const float* __restrict__ a, int lo, int hi) {
  if constexpr (U == 1) {
    float mx = -__builtin_inff();
    for (int i = lo + (int)threadIdx.x; i < hi; i += TB) mx = max_nan(mx, a[i]);
    return mx;
  } else {
    float r[U];
#pragma unroll
    for (int u = 0; u < U; ++u) r[u] = -__builtin_inff();
    for (int64_t i = lo + (int64_t)threadIdx.x; i < hi; i += (int64_t)U * TB)
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (i + (int64_t)u * TB < hi) r[u] = max_nan(r[u], a[i + (int64_t)u * TB]);
#pragma unroll
    for (int h = U / 2; h >= 1; h /= 2)
#pragma unroll
      for (int u = 0; u < h; ++u) r[u] = max_nan(r[u], r[u + h]);
    return r[0];
  }
}

template <int TB, int U>
__device__ __forceinline__ void thread_seg_sums(const double* __restrict__ a,
                                                const double* __restrict__ b, int lo, int hi,
                                                double& A, double& B) {
  if constexpr (U == 1) {
    for (int i = lo + (int)threadIdx.x; i < hi; i += TB) {
      A += a[i];
      B += b[i];
    }
  } else {
    double ra[U], rb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) ra[u] = rb[u] = 0.0;
    for (int64_t i = lo + (int64_t)threadIdx.x; i < hi; i += (int64_t)U * TB)
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (i + (int64_t)u * TB < hi) {
          ra[u] += a[i + (int64_t)u * TB];
          rb[u] += b[i + (int64_t)u * TB];
        }
#pragma unroll
    for (int h = U / 2; h >= 1; h /= 2)
#pragma unroll
      for (int u = 0; u < h; ++u) {
        ra[u] += ra[u + h];
        rb[u] += rb[u + h];
      }
    A += ra[0];
    B += rb[0];
  }
}

// Per tensor: rho = max of its segments (or, RN, the ratio of the norms from
// the segments' double sums), soft thresholds, c.  One workgroup of TB
// threads per tensor; U loads in flight per thread (thread_seg_max).
template <int TB, bool RN = false, int U = 1>
__global__ void __launch_bounds__(TB)
k_rescale_finalize(DevTable tab, const float* __restrict__ seg_max, const double* __restrict__ seg_z,
                   const double* __restrict__ seg_f, const float* __restrict__ c_avg,
                   float* __restrict__ f_prev, float* __restrict__ c_layer, float* __restrict__ c_out,
                   Coef cf, int32_t* status) {
  __shared__ float red[TB / 64];
  __shared__ double dred[2 * (TB / 64)];
  const int l = blockIdx.x;
  const int lo = tab.lseg[l];
  const int hi = tab.lseg[l + 1];
  float mx;
  if constexpr (RN) {
    double Z = 0.0, F = 0.0;
    thread_seg_sums<TB, U>(seg_z, seg_f, lo, hi, Z, F);
    block_sum2<TB>(Z, F, dred);
    mx = (Z == 0.0 || F == 0.0) ? 1.0f : (float)(__builtin_sqrt(Z) / __builtin_sqrt(F));
  } else {
    mx = thread_seg_max<TB, U>(seg_max, lo, hi);
    mx = block_max<TB>(mx, red);
  }
  if (threadIdx.x == 0) {
    const float fp = f_prev[l];
    float f = fminf(fminf(mx, cf.f_max), cf.kp * fp);
    f = fmaxf(fmaxf(f, cf.f_min), cf.km * fp);
    f_prev[l] = f;
    const float c = c_avg[l] * f;
    c_layer[l] = c;
    if (c_out) c_out[l] = c;
    if (!__builtin_isfinite(mx)) flag(status, 8);
  }
}

// Per-element step size lr*c_l for the chunk's elements.
template <int C, bool TAIL, int SPT = kSlots<C>>
__device__ __forceinline__ void step_sizes(const DevTable& tab, int64_t k, int64_t base,
                                           const float* __restrict__ c_layer, float lr,
                                           SlotsN<SPT>& st) {
  constexpr int T = Geo<C, SPT>::T;
  const int l0 = tab.l0[k];
  const int l1 = tab.l1[k];
  const float s0 = lr * c_layer[l0];
#pragma unroll
  for (int a = 0; a < SPT; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) st[a][c] = s0;
  if (l0 != l1) {
#pragma unroll
    for (int a = 0; a < SPT; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int64_t gi = base + 4 * ((int)threadIdx.x + T * a) + c;
        st[a][c] = lr * c_layer[tensor_of(tab, l0, l1, gi)];
      }
  }
}

// Compression step, pass B: x update with the per-tensor c, m = mhat (m may
// be NULL: packed momentum, the server's packed chunk is the state).
template <int C, bool TAIL, bool NT>
__device__ __forceinline__ void pass_b_chunk(int64_t kk, const DevTable& tab,
                                             const uint32_t* __restrict__ bits_s,
                                             const float* __restrict__ scales_s,
                                             const float* __restrict__ v_frozen,
                                             float* __restrict__ x, float* __restrict__ m,
                                             const float* __restrict__ c_layer, const Coef& cf) {
  const ChunkAt<C, TAIL> ch(kk, tab.N);
  const float s = scales_s[ch.k];
  uint32_t nib[kSlots<C>];
  load_sign_nibbles<C>(bits_s + ch.k * Geo<C>::WORDS, nib);
  SlotsOf<C> vz, xx, mh, st;
  load_chunk<C, TAIL, NT>(v_frozen, ch.base, ch.nk, vz);
  load_chunk<C, TAIL, NT>(x, ch.base, ch.nk, xx);
  step_sizes<C, TAIL>(tab, ch.k, ch.base, c_layer, cf.lr, st);
#pragma unroll
  for (int a = 0; a < kSlots<C>; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      mh[a][c] = signed_scale(nib, a, c, s);
      const float d = mh[a][c] / (__builtin_sqrtf(vz[a][c]) + cf.eta);
      xx[a][c] = cf.wd != 0.0f ? xx[a][c] - (st[a][c] * (d + (cf.wd * xx[a][c])))
                               : xx[a][c] - (st[a][c] * d);
    }
  store_chunk<C, TAIL, NT>(x, ch.base, ch.nk, xx);
  if (m) store_chunk<C, TAIL, NT>(m, ch.base, ch.nk, mh);  // NULL: packed momentum
}

template <int C, bool NT = false>
__global__ void __launch_bounds__(Geo<C>::T)
k_compressed_pass_b(int64_t n_full, DevTable tab, const uint32_t* __restrict__ bits_s,
                    const float* __restrict__ scales_s, const float* __restrict__ v_frozen,
                    float* __restrict__ x, float* __restrict__ m, const float* __restrict__ c_layer,
                    Coef cf) {
  const int64_t has_tail = tab.K - n_full;
  if (has_tail && blockIdx.x == 0)
    pass_b_chunk<C, true, NT>(n_full, tab, bits_s, scales_s, v_frozen, x, m, c_layer, cf);
  else
    pass_b_chunk<C, kSmall<C>, NT>((int64_t)blockIdx.x - has_tail, tab, bits_s, scales_s, v_frozen, x,
                               m, c_layer, cf);
}

// Warmup pass 1: mean gradient, moments, per-(chunk, tensor) sums of x^2 and
// u^2 in double.  NT: streaming accesses; WPE: minimum waves per SIMD.  XS:
// the sums of x^2 are carried over from the previous step's pass 2 (x_sq),
// so x is not read and only the sums of u^2 are formed (the host selects it
// only without weight decay, where u does not depend on x).  SPT: float4
// slots per thread (the workgroup is C / (4*SPT) threads); both passes take
// the same SPT, so that the sums of x^2 pass 2 carries are the ones pass 1
// would form.  DEPTH: gradients in flight while the running sum takes the
// next one.
template <int C, bool TAIL, bool NT, bool XS, int SPT, int DEPTH>
__device__ __forceinline__ void warmup_pass1_chunk(int64_t k, const DevTable& tab, int W,
                                                   const Workers& wk, const float* __restrict__ x,
                                                   float* __restrict__ m, float* __restrict__ v,
                                                   double* __restrict__ seg_x,
                                                   double* __restrict__ seg_u, const Coef& cf,
                                                   double* red) {
  const ChunkAt<C, TAIL> ch(k, tab.N);
  const int64_t base = ch.base;
  const int nk = ch.nk;
  // The gradients are summed in worker order, gradient w + 1 .. w + DEPTH
  // in flight (q[0] .. q[DEPTH-1]) while gradient w is added; m and v are
  // loaded as soon as the last gradient has been asked for.
  SlotsN<SPT> gs, mm, vv, u, xx;
  SlotsN<SPT> q[DEPTH];
  load_chunk<C, TAIL, NT, SPT>(wk.g[0], base, nk, gs);
#pragma unroll
  for (int d = 0; d < DEPTH; ++d)
    if (1 + d < W) load_chunk<C, TAIL, NT, SPT>(wk.g[1 + d], base, nk, q[d]);
  if (W <= DEPTH) {
    load_chunk<C, TAIL, NT, SPT>(m, base, nk, mm);
    load_chunk<C, TAIL, NT, SPT>(v, base, nk, vv);
  }
  for (int w = 1; w < W; ++w) {
    SlotsN<SPT> g;
#pragma unroll
    for (int a = 0; a < SPT; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) g[a][c] = q[0][a][c];
#pragma unroll
    for (int d = 0; d + 1 < DEPTH; ++d)
#pragma unroll
      for (int a = 0; a < SPT; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c) q[d][a][c] = q[d + 1][a][c];
    if (w + DEPTH < W) {
      load_chunk<C, TAIL, NT, SPT>(wk.g[w + DEPTH], base, nk, q[DEPTH - 1]);
    } else if (w + DEPTH == W) {
      load_chunk<C, TAIL, NT, SPT>(m, base, nk, mm);
      load_chunk<C, TAIL, NT, SPT>(v, base, nk, vv);
    }
#pragma unroll
    for (int a = 0; a < SPT; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) gs[a][c] = gs[a][c] + g[a][c];
  }
  if constexpr (XS) {
#pragma unroll
    for (int a = 0; a < SPT; ++a)
#pragma unroll
      for (int c = 0; c < 4; ++c) xx[a][c] = 0.0f;  // not read: weight decay is 0 here
  } else {
    load_chunk<C, TAIL, NT, SPT>(x, base, nk, xx);
  }
  const float fW = (float)W;
#pragma unroll
  for (int a = 0; a < SPT; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float gb = gs[a][c] / fW;
      mm[a][c] = (cf.beta1 * mm[a][c]) + (cf.a1 * gb);
      vv[a][c] = (cf.beta2 * vv[a][c]) + (cf.a2 * (gb * gb));
      u[a][c] = warmup_dir(mm[a][c], vv[a][c], xx[a][c], cf);
    }
  store_chunk<C, TAIL, NT, SPT>(m, base, nk, mm);
  store_chunk<C, TAIL, NT, SPT>(v, base, nk, vv);
  segment_sums<C, SPT, !XS, true>(tab, ch.k, base, nk, xx, u, red, seg_x, seg_u);
}

template <int C, bool NT = false, int WPE = 1, bool XS = false, int SPT = kSlots<C>, int DEPTH = 1>
__global__ void __launch_bounds__((Geo<C, SPT>::T), WPE)
k_warmup_pass1(int64_t n_full, DevTable tab, int W, Workers wk, const float* __restrict__ x,
               float* __restrict__ m, float* __restrict__ v, double* __restrict__ seg_x,
               double* __restrict__ seg_u, Coef cf) {
  __shared__ double red[2 * (Geo<C, SPT>::T / 64)];
  const int64_t has_tail = tab.K - n_full;
  if (has_tail && blockIdx.x == 0)
    warmup_pass1_chunk<C, true, NT, XS, SPT, DEPTH>(n_full, tab, W, wk, x, m, v, seg_x, seg_u,
                                                    cf, red);
  else
    warmup_pass1_chunk<C, Geo<C, SPT>::SMALL, NT, XS, SPT, DEPTH>((int64_t)blockIdx.x - has_tail, tab, W,
                                                         wk, x, m, v, seg_x, seg_u, cf, red);
}

// Per tensor: norms, trust ratio, clip, c_sum.  One workgroup of TB threads
// per tensor; UL loads in flight per thread (thread_seg_sums).
template <int TB, int UL = 1>
__global__ void __launch_bounds__(TB)
k_warmup_finalize(DevTable tab, const double* __restrict__ seg_x, const double* __restrict__ seg_u,
                  float* __restrict__ c_sum, float* __restrict__ c_layer, float* __restrict__ c_out,
                  Coef cf, int32_t* status) {
  __shared__ double red[2 * (TB / 64)];
  const int l = blockIdx.x;
  const int lo = tab.lseg[l];
  const int hi = tab.lseg[l + 1];
  double X = 0.0, U = 0.0;
  thread_seg_sums<TB, UL>(seg_x, seg_u, lo, hi, X, U);
  block_sum2<TB>(X, U, red);
  if (threadIdx.x == 0) {
    const float r = (X == 0.0 || U == 0.0) ? 1.0f : (float)(__builtin_sqrt(X) / __builtin_sqrt(U));
    const float c = fminf(fmaxf(r, cf.c_min), cf.c_max);
    c_sum[l] = cf.cd > 0.0f ? (cf.cd * c_sum[l]) + (cf.cd1 * c) : c_sum[l] + c;
    c_layer[l] = c;
    if (c_out) c_out[l] = c;
    if (!__builtin_isfinite(X) || !__builtin_isfinite(U)) flag(status, 4);
  }
}

// Warmup pass 2: x = x - (lr*c_l)*u with u recomputed from the new m, v.
// XO: also the per-(chunk, tensor) sums of the updated x^2 into x_sq, by the
// reduction pass 1 uses (same SPT), for the next step's pass 1 to take
// instead of reading x.
template <int C, bool TAIL, bool NT, bool XO, int SPT>
__device__ __forceinline__ void warmup_pass2_chunk(int64_t k, const DevTable& tab,
                                                   const float* __restrict__ m,
                                                   const float* __restrict__ v,
                                                   float* __restrict__ x,
                                                   const float* __restrict__ c_layer,
                                                   double* __restrict__ x_sq, const Coef& cf,
                                                   double* red) {
  const ChunkAt<C, TAIL> ch(k, tab.N);
  SlotsN<SPT> mm, vv, xx, st;
  load_chunk<C, TAIL, NT, SPT>(m, ch.base, ch.nk, mm);
  load_chunk<C, TAIL, NT, SPT>(v, ch.base, ch.nk, vv);
  load_chunk<C, TAIL, NT, SPT>(x, ch.base, ch.nk, xx);
  step_sizes<C, TAIL, SPT>(tab, ch.k, ch.base, c_layer, cf.lr, st);
#pragma unroll
  for (int a = 0; a < SPT; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float u = warmup_dir(mm[a][c], vv[a][c], xx[a][c], cf);
      xx[a][c] = xx[a][c] - (st[a][c] * u);
    }
  store_chunk<C, TAIL, NT, SPT>(x, ch.base, ch.nk, xx);
  if constexpr (XO) segment_sums<C, SPT, true, false>(tab, ch.k, ch.base, ch.nk, xx, xx, red, x_sq,
                                                      nullptr);
}

template <int C, bool NT = false, bool XO = false, int SPT = kSlots<C>>
__global__ void __launch_bounds__((Geo<C, SPT>::T))
k_warmup_pass2(int64_t n_full, DevTable tab, const float* __restrict__ m, const float* __restrict__ v,
               float* __restrict__ x, const float* __restrict__ c_layer, double* __restrict__ x_sq,
               Coef cf) {
  __shared__ double red[XO ? 2 * (Geo<C, SPT>::T / 64) : 1];
  const int64_t has_tail = tab.K - n_full;
  if (has_tail && blockIdx.x == 0)
    warmup_pass2_chunk<C, true, NT, XO, SPT>(n_full, tab, m, v, x, c_layer, x_sq, cf, red);
  else
    warmup_pass2_chunk<C, Geo<C, SPT>::SMALL, NT, XO, SPT>((int64_t)blockIdx.x - has_tail, tab, m, v, x,
                                                  c_layer, x_sq, cf, red);
}

// Freeze, element part: v_fresh = v, error buffers cleared.
template <int C, bool TAIL>
__device__ __forceinline__ void freeze_elems_chunk(int64_t k, int64_t n, int W,
                                                   const float* __restrict__ v,
                                                   float* __restrict__ v_fresh, const Workers& wk,
                                                   float* __restrict__ err_s) {
  const ChunkAt<C, TAIL> ch(k, n);
  SlotsOf<C> vv, zero;
  load_chunk<C, TAIL>(v, ch.base, ch.nk, vv);
  store_chunk<C, TAIL>(v_fresh, ch.base, ch.nk, vv);
#pragma unroll
  for (int a = 0; a < kSlots<C>; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) zero[a][c] = 0.0f;
  for (int w = 0; w < W; ++w) store_chunk<C, TAIL>(wk.e[w], ch.base, ch.nk, zero);
  store_chunk<C, TAIL>(err_s, ch.base, ch.nk, zero);
}

template <int C>
__global__ void __launch_bounds__(Geo<C>::T)
k_freeze_elems(int64_t n_full, int64_t n, int W, const float* __restrict__ v,
               float* __restrict__ v_fresh, Workers wk, float* __restrict__ err_s) {
  const int64_t has_tail = partial_chunks<C>(n_full, n);
  if (has_tail && blockIdx.x == 0)
    freeze_elems_chunk<C, true>(n_full, n, W, v, v_fresh, wk, err_s);
  else
    freeze_elems_chunk<C, kSmall<C>>((int64_t)blockIdx.x - has_tail, n, W, v, v_fresh, wk, err_s);
}

// Freeze, tensor part: c_avg = c_sum / den (den = T_w, or 1-d^T_w for the
// EMA variant), f_prev = 1.
__global__ void __launch_bounds__(256)
k_freeze_tensors(int L, const float* __restrict__ c_sum, float Tw, float* __restrict__ c_avg,
                 float* __restrict__ f_prev) {
  const int l = blockIdx.x * 256 + threadIdx.x;
  if (l < L) {
    c_avg[l] = c_sum[l] / Tw;
    f_prev[l] = 1.0f;
  }
}

}  // namespace onebit
