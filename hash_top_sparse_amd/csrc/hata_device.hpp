// hata_device.hpp -- device helpers shared by the HATA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hata {

constexpr int kD = 128;      // head dim
constexpr int kR = 128;      // default code bits
constexpr int kWords32 = 4;  // 32-bit words per default code
constexpr int kNT = 256;     // threads per workgroup of the decode kernels

// Code widths: a code row of R bits is stored as R/32 32-bit words, bit c in
// bit c % 32 of word c / 32 (4 bytes at R = 32; for R >= 64 the same bytes as
// R/64 little-endian 64-bit words).  W64 is the 64-bit word count of the
// LDS layout the projection writes.
template <int R>
struct Width {
  static_assert(R == 32 || R == 64 || R == 128 || R == 256, "code width");
  static constexpr int W64 = (R + 63) / 64;  // 64-bit words per row in LDS (bits past R zero)
  static constexpr int W32 = (R + 31) / 32;  // 32-bit words per stored code row
  static constexpr int CPT = R / 32;         // projection columns per thread
};

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_lo(uint32_t two) { return __uint_as_float(two << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t two) { return __uint_as_float(two & 0xFFFF0000u); }

// 8 bf16 (one 16-byte load) -> 8 fp32
__device__ __forceinline__ void unpack8(const uint4 v, float (&f)[8]) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
  f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
  f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

// ------------------------------------------------------- memory access
// Streaming 16-byte load that should not displace reusable lines.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 load_stream16(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 load_stream8(const uint2* p) {
  const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint32_t load_stream4(const uint32_t* p) { return __builtin_nontemporal_load(p); }

// Agent-coherent accesses for data that workgroups of one launch exchange.
// They compile to global_load/global_store with the device-scope cache bit
// (sc1), which bypasses the per-XCD L2 state that another XCD cannot see,
// so no L2 writeback or invalidate is needed around them.
template <typename T>
__device__ __forceinline__ void st_agent(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T ld_agent(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wide agent-coherent access to a workspace exchange area through a buffer
// resource: 16-byte loads/stores with the device-scope bit, bounds-checked by
// the hardware against `bytes` (out-of-range loads return 0, stores drop).
constexpr int kSC1 = 16;  // cache-policy bit: device-scope coherence
struct CohBuf {
  __amdgpu_buffer_rsrc_t r;
  __device__ __forceinline__ CohBuf(const void* base, uint32_t bytes)
      : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000)) {}
  __device__ __forceinline__ u32x4 ld16(uint32_t off) const {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kSC1);
  }
  __device__ __forceinline__ void st16(uint32_t off, u32x4 v) const {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, kSC1);
  }
  // Stores for an exchange whose readers all run on the writer's XCD: a
  // plain store lands in that XCD's L2, where the readers' sc1 loads find it
  // (it is not written through to memory, so the ack comes sooner).
  __device__ __forceinline__ void st16x(uint32_t off, u32x4 v, bool xcd_local) const {
    if (xcd_local) __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, 0);
    else __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, kSC1);
  }
  __device__ __forceinline__ void st4x(uint32_t off, uint32_t v, bool xcd_local) const {
    if (xcd_local) __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)off, 0, 0);
    else __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)off, 0, kSC1);
  }
  __device__ __forceinline__ uint32_t ld4(uint32_t off) const {
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, kSC1);
  }
  __device__ __forceinline__ void st4(uint32_t off, uint32_t v) const {
    __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)off, 0, kSC1);
  }
};

// Wait until every memory operation this wave issued has completed.
__device__ __forceinline__ void wait_all_mem() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ------------------------------------------------------- wave reductions
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// Sum over each aligned group of 16 lanes; every lane gets the group's sum.
// quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror.
__device__ __forceinline__ float sum16(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  v += dpp_f<0x140>(v);
  return v;
}

template <int CTRL, int ROW_MASK, bool BOUND_ZERO>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return __builtin_amdgcn_update_dpp(0u, v, CTRL, ROW_MASK, 0xF, BOUND_ZERO);
}
// Inclusive prefix sum over the 64 lanes of a wave: row_shr 1/2/4/8 within
// each row of 16 lanes, then row_bcast15 and row_bcast31 carry the row totals.
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v) {
  v += dpp_u<0x111, 0xF, true>(v);
  v += dpp_u<0x112, 0xF, true>(v);
  v += dpp_u<0x114, 0xF, true>(v);
  v += dpp_u<0x118, 0xF, true>(v);
  v += dpp_u<0x142, 0xA, false>(v);
  v += dpp_u<0x143, 0xC, false>(v);
  return v;
}
// Sum over the 64 lanes of a wave (every lane gets the total).
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  return __builtin_amdgcn_readlane(wave_incl_scan_u32(v), 63);
}
// Values of lanes l and l^32 (resp. l^16), as (bit clear, bit set); both
// lanes of a pair see the same two values, so pair results are identical.
__device__ __forceinline__ float pair32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair16_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ int pair32_min_i(int v) {
  const auto r = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
  return min((int)r[0], (int)r[1]);
}
__device__ __forceinline__ int pair16_min_i(int v) {
  const auto r = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
  return min((int)r[0], (int)r[1]);
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_fm(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(-INFINITY), __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// Maximum within each row of 16 lanes (every lane of the row gets it).
__device__ __forceinline__ float row16_max_f(float v) {
  v = fmaxf(v, dpp_fm<0xB1>(v));
  v = fmaxf(v, dpp_fm<0x4E>(v));
  v = fmaxf(v, dpp_fm<0x141>(v));
  v = fmaxf(v, dpp_fm<0x140>(v));
  return v;
}
// Minimum over the 64 lanes of a wave (every lane gets it).
__device__ __forceinline__ int wave_min_i(int v) {
  v = min(v, dpp_i<0xB1>(v));
  v = min(v, dpp_i<0x4E>(v));
  v = min(v, dpp_i<0x141>(v));
  v = min(v, dpp_i<0x140>(v));
  v = pair16_min_i(v);
  return pair32_min_i(v);
}

// Exclusive scan over the 256 threads of a workgroup; `tmp` holds 4 words of
// LDS.  Returns the exclusive prefix; *total gets the block sum.  Contains
// __syncthreads, so every thread must call it.
__device__ __forceinline__ uint32_t block_excl_scan_u32(uint32_t v, uint32_t* tmp, uint32_t* total) {
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  (void)lane;
  uint32_t inc = wave_incl_scan_u32(v);
  if (lane == 63) tmp[wv] = inc;
  __syncthreads();
  uint32_t base = 0, all = 0;
#pragma unroll
  for (int i = 0; i < kNT / 64; ++i) {
    uint32_t s = tmp[i];
    base += (i < wv) ? s : 0u;
    all += s;
  }
  __syncthreads();
  *total = all;
  return base + inc - v;
}

// ------------------------------------------------------- HashEncode projection
// Projection of ROWS staged rows by one KV head's W_H ([128][R] fp32,
// row-major) with a 256-thread workgroup, then sign + bit-pack:
//   thread t owns columns CPT*(t&31) .. +CPT-1 (CPT = R/32) and input
//   channels 16*(t>>5) .. +15 (16*CPT floats of W per thread); partial sums
//   over its 16 channels are added pairwise across the two channel groups of
//   a wave (lanes l, l^32), then over the 4 waves in fixed order through
//   LDS; each 64-column word of a code is one wave64 ballot of (p >= 0)
//   (for R = 32 the lanes past column 31 vote 0).
// The summation order is fixed, so every kernel that uses this function
// produces identical codes.
template <int R = kR>
struct WRegs {
  float w[16][Width<R>::CPT];
};
template <int R = kR>
__device__ __forceinline__ void load_w_regs(const float* __restrict__ Wh, WRegs<R>& wr) {
  constexpr int CPT = Width<R>::CPT;
  const int t = threadIdx.x, cg = t & 31, rg = t >> 5;
  const float* src = Wh + (rg * 16) * R + cg * CPT;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if constexpr (CPT == 8) {
      const float4 a = reinterpret_cast<const float4*>(src + i * R)[0];
      const float4 b = reinterpret_cast<const float4*>(src + i * R)[1];
      wr.w[i][0] = a.x; wr.w[i][1] = a.y; wr.w[i][2] = a.z; wr.w[i][3] = a.w;
      wr.w[i][4] = b.x; wr.w[i][5] = b.y; wr.w[i][6] = b.z; wr.w[i][7] = b.w;
    } else if constexpr (CPT == 4) {
      const float4 a = *reinterpret_cast<const float4*>(src + i * R);
      wr.w[i][0] = a.x; wr.w[i][1] = a.y; wr.w[i][2] = a.z; wr.w[i][3] = a.w;
    } else if constexpr (CPT == 2) {
      const float2 a = *reinterpret_cast<const float2*>(src + i * R);
      wr.w[i][0] = a.x; wr.w[i][1] = a.y;
    } else {
      wr.w[i][0] = src[i * R];
    }
  }
}
// xs: LDS rows [ROWS][128] fp32; red: LDS [4][ROWS][R] fp32; out: LDS
// [ROWS][W64] uint64.  Rows >= nrows are not packed (their products are
// formed and dropped, so they may hold anything).  The FMA loop runs over
// W's registers in load order, all rows at once, so the products with the
// first W registers start while the later ones are still arriving; each
// accumulator still takes its 16 channels in ascending order.  Ends with
// __syncthreads.
template <int ROWS, int R = kR>
__device__ __forceinline__ void project_pack(const WRegs<R>& wr, const float* xs, float* red,
                                             uint64_t* out, int nrows) {
  constexpr int CPT = Width<R>::CPT, W64 = Width<R>::W64;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6, cg = t & 31, rg = t >> 5;
  float acc[ROWS][CPT];
#pragma unroll
  for (int r = 0; r < ROWS; ++r)
#pragma unroll
    for (int c = 0; c < CPT; ++c) acc[r][c] = 0.f;
#pragma unroll
  for (int i4 = 0; i4 < 4; ++i4) {
    float4 xq[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) xq[r] = reinterpret_cast<const float4*>(xs + r * kD + rg * 16)[i4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int r = 0; r < ROWS; ++r) {
        const float xv = (j == 0) ? xq[r].x : (j == 1) ? xq[r].y : (j == 2) ? xq[r].z : xq[r].w;
#pragma unroll
        for (int c = 0; c < CPT; ++c) acc[r][c] = fmaf(xv, wr.w[i4 * 4 + j][c], acc[r][c]);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < ROWS; ++r) {
    if (r >= nrows) break;
    float sv[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) sv[c] = pair32_sum(acc[r][c]);
    if (lane < 32) {
      float* dst = red + (wv * ROWS + r) * R + cg * CPT;
      if constexpr (CPT == 8) {
        reinterpret_cast<float4*>(dst)[0] = make_float4(sv[0], sv[1], sv[2], sv[3]);
        reinterpret_cast<float4*>(dst)[1] = make_float4(sv[4], sv[5], sv[6], sv[7]);
      } else if constexpr (CPT == 4) {
        *reinterpret_cast<float4*>(dst) = make_float4(sv[0], sv[1], sv[2], sv[3]);
      } else if constexpr (CPT == 2) {
        *reinterpret_cast<float2*>(dst) = make_float2(sv[0], sv[1]);
      } else {
        dst[0] = sv[0];
      }
    }
  }
  __syncthreads();
  // (row, word) pair p = row * W64 + word goes to wave p % 4
#pragma unroll
  for (int p = wv; p < ROWS * W64; p += 4) {
    const int r = p / W64, wd = p - r * W64;
    if (r >= nrows) break;
    const int col = wd * 64 + lane;
    const int cc = col < R ? col : R - 1;
    float s = red[(0 * ROWS + r) * R + cc];
    s += red[(1 * ROWS + r) * R + cc];
    s += red[(2 * ROWS + r) * R + cc];
    s += red[(3 * ROWS + r) * R + cc];
    const uint64_t m = __ballot(col < R && s >= 0.0f);
    if (lane == 0) out[p] = m;
  }
  __syncthreads();
}

// ------------------------------------------------------- Hamming with GQA sum
// For a code c and G query codes q_g, sum_g popcount(q_g ^ c) equals
// sum over bits of (c_bit ? #{g : q_g bit = 0} : #{g : q_g bit = 1}).  Both
// per-bit counts are kept bit-sliced (J slices of 32-bit masks per word), so
// the per-token work is J bitfield-selects and J popcounts per word instead
// of G xors and G popcounts.
template <int G>
struct SliceCount {
  static constexpr int J = (G == 1) ? 1 : (G == 2) ? 2 : (G <= 7) ? 3 : 4;
};

template <int G, int R = kR>
struct QMasks {
  uint32_t one[SliceCount<G>::J][Width<R>::W32];   // bit slices of #{g: q_g bit = 1}
  uint32_t zero[SliceCount<G>::J][Width<R>::W32];  // bit slices of #{g: q_g bit = 0}
};

// qw[g][w]: 32-bit word w of query code g.
template <int G, int R = kR>
__device__ __forceinline__ void build_qmasks(const uint32_t (&qw)[G][Width<R>::W32], QMasks<G, R>& m) {
  constexpr int J = SliceCount<G>::J;
#pragma unroll
  for (int w = 0; w < Width<R>::W32; ++w) {
    uint32_t c1[J], c0[J];
#pragma unroll
    for (int j = 0; j < J; ++j) { c1[j] = 0; c0[j] = 0; }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      uint32_t x1 = qw[g][w], x0 = ~qw[g][w];
#pragma unroll
      for (int j = 0; j < J; ++j) {  // bit-sliced increment by one bit
        uint32_t n1 = c1[j] ^ x1, n0 = c0[j] ^ x0;
        x1 &= c1[j];
        x0 &= c0[j];
        c1[j] = n1;
        c0[j] = n0;
      }
    }
#pragma unroll
    for (int j = 0; j < J; ++j) { m.one[j][w] = c1[j]; m.zero[j][w] = c0[j]; }
  }
}

// summed distance of one code (its W32 32-bit words) to the G query codes
template <int G, int R>
__device__ __forceinline__ uint32_t gqa_hamming_w(const uint32_t (&cw)[Width<R>::W32], const QMasks<G, R>& m) {
  constexpr int J = SliceCount<G>::J;
  uint32_t s = 0;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    uint32_t acc = 0;
#pragma unroll
    for (int w = 0; w < Width<R>::W32; ++w) {
      uint32_t sel = (cw[w] & m.zero[j][w]) | (~cw[w] & m.one[j][w]);
      acc = __builtin_popcount(sel) + acc;
    }
    s += acc << j;
  }
  return s;
}

template <int G>
__device__ __forceinline__ uint32_t gqa_hamming(const uint4 c, const QMasks<G>& m) {
  const uint32_t cw[4] = {c.x, c.y, c.z, c.w};
  return gqa_hamming_w<G, kR>(cw, m);
}

// One code row of R bits as loaded by the scans: 4, 8, 16 or 32 bytes.
template <int R>
struct CodeRow {
  uint4 v[(Width<R>::W32 + 3) / 4];
};
// streaming load of code row `row` (R/8 bytes) from codes
template <int R>
__device__ __forceinline__ CodeRow<R> load_code(const uint32_t* codes, int64_t row) {
  CodeRow<R> c;
  if constexpr (Width<R>::W32 == 1) {
    c.v[0] = make_uint4(load_stream4(codes + row), 0u, 0u, 0u);
  } else if constexpr (Width<R>::W32 == 2) {
    const uint2 v = load_stream8(reinterpret_cast<const uint2*>(codes + row * 2));
    c.v[0] = make_uint4(v.x, v.y, 0u, 0u);
  } else {
#pragma unroll
    for (int i = 0; i < Width<R>::W32 / 4; ++i)
      c.v[i] = load_stream16(reinterpret_cast<const uint4*>(codes + row * Width<R>::W32) + i);
  }
  return c;
}
// 32-bit word wd of a code row held as 64-bit words (the projection's layout)
__device__ __forceinline__ uint32_t code_word32(const uint64_t* row64, int wd) {
  return (uint32_t)(row64[wd >> 1] >> ((wd & 1) * 32));
}
template <int R>
__device__ __forceinline__ void code_words(const CodeRow<R>& c, uint32_t (&cw)[Width<R>::W32]) {
  if constexpr (Width<R>::W32 <= 2) {
    cw[0] = c.v[0].x;
    if constexpr (Width<R>::W32 == 2) cw[1] = c.v[0].y;
  } else {
#pragma unroll
    for (int i = 0; i < Width<R>::W32 / 4; ++i) {
      cw[4 * i] = c.v[i].x; cw[4 * i + 1] = c.v[i].y; cw[4 * i + 2] = c.v[i].z; cw[4 * i + 3] = c.v[i].w;
    }
  }
}

// ------------------------------------------------------- online softmax
// Per-lane state of a 16-lane group that attends rows with G query heads;
// the lane holds 8 of the 128 channels (channels sub*8 .. sub*8+7).
template <int G>
struct SoftmaxState {
  float m[G], l[G], acc[G][8];
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      m[g] = -INFINITY;
      l[g] = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[g][c] = 0.f;
    }
  }
};

// Attend UNROLL rows at once: logits, one max update, then weights.  `valid`
// masks rows past the end (their loads must not have been issued).
template <int G, int UNROLL>
__device__ __forceinline__ void attend_block(SoftmaxState<G>& st, const float (&qreg)[G][8],
                                             const uint4 (&kv)[UNROLL], const uint4 (&vv)[UNROLL],
                                             const bool (&valid)[UNROLL], float scale) {
  float z[UNROLL][G];
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) {
    float kf[8];
    unpack8(kv[u], kf);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < 8; ++c) s = fmaf(qreg[g][c], kf[c], s);
      z[u][g] = sum16(s) * scale;
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float mx = st.m[g];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) mx = valid[u] ? fmaxf(mx, z[u][g]) : mx;
    // exp(-inf) = 0 when m was -inf; no valid row at all keeps the state
    const float alpha = (mx == -INFINITY) ? 1.f : __expf(st.m[g] - mx);
    st.l[g] *= alpha;
#pragma unroll
    for (int c = 0; c < 8; ++c) st.acc[g][c] *= alpha;
    st.m[g] = mx;
  }
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) {
    if (!valid[u]) continue;
    float vf[8];
    unpack8(vv[u], vf);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float p = __expf(z[u][g] - st.m[g]);
      st.l[g] += p;
#pragma unroll
      for (int c = 0; c < 8; ++c) st.acc[g][c] = fmaf(p, vf[c], st.acc[g][c]);
    }
  }
}

// Merge the 16 row-group states of a 256-thread workgroup (4 waves x 4
// groups of 16 lanes) into one (M, L, A[128]) record per head:
//   step 1 combines the 4 groups of a wave with xor-shuffles over 16 and 32
//   lanes; step 2 combines the 4 waves through LDS.
// red: LDS of kMergeFloats<G> floats, laid out [4 waves][G][2 + 128]; on
// return red[0][g] holds head g's merged record.  Fixed merge order.
constexpr int kRec = 2 + kD;
template <int G>
constexpr int kMergeFloats = 4 * G * kRec;

template <int G>
__device__ __forceinline__ void merge_wg(const SoftmaxState<G>& st, float* red) {
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6, sub = lane & 15;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float M = pair32_max(pair16_max(st.m[g]));
    const float f = (M == -INFINITY) ? 0.f : __expf(st.m[g] - M);
    const float L = pair32_sum(pair16_sum(st.l[g] * f));
    float A[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) A[c] = pair32_sum(pair16_sum(st.acc[g][c] * f));
    if (lane < 16) {
      float* r = red + (wv * G + g) * kRec;
      if (sub == 0) { r[0] = M; r[1] = L; }
#pragma unroll
      for (int c = 0; c < 8; ++c) r[2 + sub * 8 + c] = A[c];
    }
  }
  __syncthreads();
  constexpr int PER = (G * kD + kNT - 1) / kNT;
  float Ms[PER], Ls[PER], As[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = t + i * kNT;
    Ms[i] = -INFINITY; Ls[i] = 0.f; As[i] = 0.f;
    if (e >= G * kD) continue;
    const int g = e / kD, c = e % kD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, red[(w * G + g) * kRec]);
    float L = 0.f, A = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float* r = red + (w * G + g) * kRec;
        const float f = __expf(r[0] - M);
        L = fmaf(r[1], f, L);
        A = fmaf(r[2 + c], f, A);
      }
    }
    Ms[i] = M; Ls[i] = L; As[i] = A;
  }
  __syncthreads();  // every wave record has been read
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = t + i * kNT;
    if (e >= G * kD) continue;
    const int g = e / kD, c = e % kD;
    float* r0 = red + g * kRec;
    if (c == 0) { r0[0] = Ms[i]; r0[1] = Ls[i]; }
    r0[2 + c] = As[i];
  }
  __syncthreads();
}

// End of the attention: merge the 4 row groups of each wave (permlane
// swaps), then, when several waves share a head, the waves in fixed order
// through LDS.  Writes red[g*kRec + {M, L, A[128]}]; ends with
// __syncthreads.
template <int G>
__device__ __forceinline__ void finish_heads(const SoftmaxState<(G >= 4) ? G / 4 : 1>& st, float* red) {
  constexpr int HPW = (G >= 4) ? G / 4 : 1;
  constexpr int WPH = (G >= 4) ? 1 : 4 / G;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6, rg = lane >> 4, sub = lane & 15;
  const int hg = wv / WPH;
  const int g0 = hg * HPW;
  float* tmp = red + G * kRec;  // [4 waves][kRec] when several waves share a head
#pragma unroll
  for (int i = 0; i < HPW; ++i) {
    const float M = pair32_max(pair16_max(st.m[i]));
    const float f = (M == -INFINITY) ? 0.f : __expf(st.m[i] - M);
    const float L = pair32_sum(pair16_sum(st.l[i] * f));
    float A[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) A[c] = pair32_sum(pair16_sum(st.acc[i][c] * f));
    if (rg == 0) {
      float* r = (WPH == 1) ? red + (g0 + i) * kRec : tmp + wv * kRec;
      if (sub == 0) { r[0] = M; r[1] = L; }
#pragma unroll
      for (int c = 0; c < 8; ++c) r[2 + sub * 8 + c] = A[c];
    }
  }
  __syncthreads();
  if (WPH > 1) {
    // merge the WPH row partitions of each head in fixed order
    for (int e = t; e < G * kD; e += kNT) {
      const int g = e / kD, c = e % kD;
      float M = -INFINITY;
      for (int p = 0; p < WPH; ++p) M = fmaxf(M, tmp[(g * WPH + p) * kRec]);
      float L = 0.f, A = 0.f;
      if (M != -INFINITY) {
        for (int p = 0; p < WPH; ++p) {
          const float* r = tmp + (g * WPH + p) * kRec;
          const float f = __expf(r[0] - M);
          L = fmaf(r[1], f, L);
          A = fmaf(r[2 + c], f, A);
        }
      }
      float* o = red + g * kRec;
      if (c == 0) { o[0] = M; o[1] = L; }
      o[2 + c] = A;
    }
    __syncthreads();
  }
}


// One query head per KV head: the 4 waves split the kept rows and no row is
// used by two waves, so nothing is staged in LDS.  The 16 groups of 16 lanes
// take rows grp, grp + 16, grp + 32, ... (grp = 4*wave + group within the
// wave); each step covers UN rows of every group, and the loads of the next
// NPF steps stay in flight in a register ring (NPF*UN*512 bytes per group).
// Row ids past the list are clamped to its last row, so every load is issued
// unconditionally (the compiler can count them exactly) and the extra rows
// are masked out of the softmax.
// Row map of the gather: cache row of a kept token (the identity for a
// contiguous cache).
struct SameRows {
  __device__ __forceinline__ int64_t operator()(int64_t tok) const { return tok; }
};
// Paged cache: token tok of KV head h lives in page pgl[tok / P - fp] (the
// page ids of a workgroup's chunk, held in LDS, all valid pool pages) of a
// pool laid out [pages][Hkv][P][128]; the LDS index is clamped into the
// list, so even a stray token id maps into the pool.
struct PagedRows {
  const int32_t* pgl;
  int fp, log2P, Hkv, h, last;
  __device__ __forceinline__ int64_t operator()(int64_t tok) const {
    const int i = min(max((int)(tok >> log2P) - fp, 0), last);
    return (((int64_t)pgl[i] * Hkv + h) << log2P) + (tok & ((int64_t(1) << log2P) - 1));
  }
};

template <int UN, int NPF, class Map = SameRows>
__device__ __forceinline__ void attend_rows_g1(const float* qf, const int32_t* sel, int m, int n,
                                               const uint16_t* K, const uint16_t* V, float scale,
                                               float* red, const Map& map = Map()) {
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6, rg = lane >> 4, sub = lane & 15;
  const int grp = wv * 4 + rg;
  float qreg[1][8];
#pragma unroll
  for (int c = 0; c < 8; ++c) qreg[0][c] = qf[sub * 8 + c];
  SoftmaxState<1> st;
  st.init();
  const int nsteps = (m + 16 * UN - 1) / (16 * UN);
  auto issue = [&](int step, uint4 (&kk)[UN], uint4 (&vv)[UN]) {
    int tok[UN];
#pragma unroll
    for (int u = 0; u < UN; ++u) tok[u] = sel[max(min((step * UN + u) * 16 + grp, m - 1), 0)];
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int64_t off = map((int64_t)min(max(tok[u], 0), n - 1)) * kD + sub * 8;
      kk[u] = *reinterpret_cast<const uint4*>(K + off);
      vv[u] = *reinterpret_cast<const uint4*>(V + off);
    }
  };
  uint4 kr[NPF][UN], vr[NPF][UN];
#pragma unroll
  for (int j = 0; j < NPF; ++j) issue(j, kr[j], vr[j]);
  for (int s0 = 0; s0 < nsteps; s0 += NPF) {
#pragma unroll
    for (int j = 0; j < NPF; ++j) {
      const int step = s0 + j;
      if (step >= nsteps) break;
      bool valid[UN];
#pragma unroll
      for (int u = 0; u < UN; ++u) valid[u] = (step * UN + u) * 16 + grp < m;
      attend_block<1, UN>(st, qreg, kr[j], vr[j], valid, scale);
      issue(step + NPF, kr[j], vr[j]);  // past the list: clamped, never used
    }
  }
  finish_heads<1>(st, red);
}

// No-op phase marker (the phase-trace build passes one that records times).
struct NoMark {
  __device__ __forceinline__ void operator()(int) const {}
};

// Attention over the kept rows on the matrix cores (G = 2, 4, 8 query heads
// per KV head; 256 threads).  Rows are taken in batches of 64 and staged in
// LDS as they come from HBM (K then V, 16-byte pieces), in 528-byte rows so
// that the 16 rows of a logit tile fall on distinct bank groups; rows past
// the list are staged as zeros, and the next batch's loads are in flight
// while a batch is used.  Per batch every wave forms the whole logit tile
// S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (keys as M in 16-key tiles,
// heads as N, the 128 channels in 4 steps of 32), so the four waves hold
// identical logits and the same running max without exchanging them.  Wave w
// then accumulates O^T = V^T P^T for channels [32 w, 32 w + 32) over steps
// of 32 keys, with the weights split into two bf16 terms P = hi + lo
// (lo = bf16(P - hi)): both contractions run on the matrix cores and the
// split leaves a relative error of at most 2^-16 in each weight.  q and K
// are bf16, so the logits' products are exact and only their fp32 summation
// order differs from a plain dot product.  The k index of the V^T P^T
// product runs over the keys in the order the S^T accumulators hold them
// (lane group h4 holds keys 4 h4 .. 4 h4 + 3 of each 16-key tile); the V^T
// operand is gathered in that order with 2-byte LDS reads.  Tiles past the
// batch are skipped by uniform branches.  Writes red[g*kRec + {M, L, A[128]}]
// (M: running max of the scaled logits, L: sum of the weights, A: weighted
// V relative to M); ends with __syncthreads.  kvl: LDS of kMxLdsBytes.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef unsigned short u16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
constexpr int kMxRows = 64;                    // kept rows per batch
constexpr int kMxRow = 2 * kD + 8;             // uint16 per staged row (K, V, 16 bytes of padding)
constexpr int kMxLdsBytes = kMxRows * kMxRow * 2;

template <int G, class Map = SameRows, class Mark = NoMark>
__device__ __forceinline__ void attend_heads_mx(const float* qf, const int32_t* sel, int m, int n,
                                                const uint16_t* K, const uint16_t* V, float scale,
                                                float* red, uint16_t* kvl, const Map& map = Map(),
                                                const Mark& mark = Mark()) {
  static_assert(G >= 2 && G <= 16, "heads are the N index of a 16-wide tile");
  constexpr int LPT = kMxRows * 32 / kNT;  // 16-byte staging loads per thread and batch
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6, h4 = lane >> 4, l16 = lane & 15;
  // staging slot i of thread t: piece c = t + 256 i, row c >> 5, 16-byte
  // part c & 31 (parts 0..15: K channels 8 p .. 8 p + 7; 16..31: V)
  auto gather = [&](int r0, uint4 (&v)[LPT]) {
    const int mb = min(kMxRows, m - r0);
    int tokv[LPT];
#pragma unroll
    for (int i = 0; i < LPT; ++i) tokv[i] = sel[r0 + max(min((t >> 5) + 8 * i, mb - 1), 0)];
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int c = t + i * kNT, r = c >> 5, part16 = c & 31;
      v[i] = make_uint4(0, 0, 0, 0);
      if (r < mb) {
        const int64_t tok = min(max(tokv[i], 0), n - 1);
        const uint16_t* src = (part16 < 16 ? K : V) + map(tok) * kD + (part16 & 15) * 8;
        v[i] = *reinterpret_cast<const uint4*>(src);
      }
    }
  };
  // B operand of S^T = K Q^T: head l16 (zero past G), channels 32 kk + 8 h4 + j
  // (every lane reads a valid row, the select follows the loads: a
  // conditional load here would be a branch and a wait per element)
  bf16x8_t qb[4];
  {
    const float* qrow = qf + min(l16, G - 1) * kD + 8 * h4;
    const bool keep = l16 < G;
    float4 qv[8];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      qv[2 * kk] = *reinterpret_cast<const float4*>(qrow + 32 * kk);
      qv[2 * kk + 1] = *reinterpret_cast<const float4*>(qrow + 32 * kk + 4);
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const float f[8] = {qv[2 * kk].x, qv[2 * kk].y, qv[2 * kk].z, qv[2 * kk].w,
                          qv[2 * kk + 1].x, qv[2 * kk + 1].y, qv[2 * kk + 1].z, qv[2 * kk + 1].w};
#pragma unroll
      for (int j = 0; j < 8; ++j) qb[kk][j] = (__bf16)(keep ? f[j] : 0.f);
    }
  }
  float m_run = -INFINITY, l_run = 0.f;
  f32x4_t o[2];
#pragma unroll
  for (int c2 = 0; c2 < 2; ++c2) o[c2] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  uint4 pv[LPT];
  gather(0, pv);
  for (int r0 = 0; r0 < m; r0 += kMxRows) {
    const int mb = min(kMxRows, m - r0);
    if (r0 > 0) __syncthreads();  // the previous batch is no longer read
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int c = t + i * kNT;
      *reinterpret_cast<uint4*>(kvl + (c >> 5) * kMxRow + (c & 31) * 8) = pv[i];
    }
    if (r0 + kMxRows < m) gather(r0 + kMxRows, pv);  // in flight while this batch is used
    __syncthreads();
    if (r0 == 0) mark(0);
    // V^T operands (A of O^T = V^T P^T) for channel tiles 2 wv + c2 and key
    // steps ps, read before the logits so that both LDS round trips overlap:
    // k index 8 h4 + j is key 32 ps + 4 h4 + j (j < 4) or 32 ps + 16 + 4 h4 + j - 4
    bf16x8_t va[2][2];
    auto load_va = [&](int ps) {
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        const uint16_t* vcol = kvl + kD + 32 * wv + 16 * c2 + l16;
        u16x8_t a16;
#pragma unroll
        for (int j = 0; j < 8; ++j) a16[j] = vcol[(32 * ps + 16 * (j >> 2) + 4 * h4 + (j & 3)) * kMxRow];
        va[ps][c2] = __builtin_bit_cast(bf16x8_t, a16);
      }
    };
    load_va(0);
    if (mb > 32) load_va(1);
    // logits: s[kt][i] is key 16 kt + 4 h4 + i of the batch for head l16
    // (channels in two independent accumulations, added at the end)
    f32x4_t s[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      s[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if (16 * kt < mb) {
        const uint16_t* krow = kvl + (16 * kt + l16) * kMxRow + 8 * h4;
        bf16x8_t ka[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) ka[kk] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(krow + 32 * kk));
        f32x4_t s2 = f32x4_t{0.f, 0.f, 0.f, 0.f};
        s[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[0], qb[0], s[kt], 0, 0, 0);
        s2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[2], qb[2], s2, 0, 0, 0);
        s[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[1], qb[1], s[kt], 0, 0, 0);
        s2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[3], qb[3], s2, 0, 0, 0);
        s[kt] += s2;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      if (16 * kt < mb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool ok = 16 * kt + 4 * h4 + i < mb;
          s[kt][i] = ok ? s[kt][i] * scale : -INFINITY;
          mx = fmaxf(mx, s[kt][i]);
        }
      }
    }
    mx = pair32_max(pair16_max(mx));  // over the batch's keys, per head
    const float m_new = fmaxf(m_run, mx);
    // exp(-inf) = 0 when m_run was -inf
    const float alpha = (m_new == -INFINITY) ? 1.f : __expf(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) o[c2] *= alpha;
    m_run = m_new;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      if (16 * kt < mb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = (16 * kt + 4 * h4 + i < mb) ? __expf(s[kt][i] - m_new) : 0.f;
          s[kt][i] = p;
          l_run += p;
        }
      } else {
        s[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    }
    // O^T += V^T P^T over steps of 32 keys (tiles 2 ps and 2 ps + 1), the
    // weights taken in the V^T operand's key order
#pragma unroll
    for (int ps = 0; ps < 2; ++ps) {
      if (32 * ps < mb) {
        bf16x8_t hi, lo;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float p = s[2 * ps + (j >> 2)][j & 3];
          const __bf16 ph = (__bf16)p;
          hi[j] = ph;
          lo[j] = (__bf16)(p - (float)ph);
        }
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          o[c2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[ps][c2], hi, o[c2], 0, 0, 0);
          o[c2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[ps][c2], lo, o[c2], 0, 0, 0);
        }
      }
    }
  }
  mark(1);
  const float L = pair32_sum(pair16_sum(l_run));
  if (l16 < G) {
    float* r = red + l16 * kRec;
    // accumulator i of channel tile 2 wv + c2 holds channel 32 wv + 16 c2 + 4 h4 + i
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
      for (int i = 0; i < 4; ++i) r[2 + 32 * wv + 16 * c2 + 4 * h4 + i] = o[c2][i];
    if (wv == 0 && h4 == 0) { r[0] = m_run; r[1] = L; }
  }
  __syncthreads();
}

}  // namespace hata
