// train.hip -- one training step of the hash weights W_H on collected Q/K.
//
// HATA notes, section "Key design", subsection "Learning-to-Hash modelling":
// the relaxed hash h(x) = 2 Sigmoid(sigma x W_H) - 1 (evaluated as
// tanh(sigma x W_H / 2), the same function), the objective
//   eps * sum_j sum_i s_ji ||h(q_j) - h(k_i)||^2      (similarity)
// + eta * sum_j ||sum_i h(k_i)||^2                      (bit balance)
// + lam * ||W_H^T W_H - I_r||_F                         (decorrelation)
// and the training pairs: each sampled query j at position p_j pairs with
// keys 0..p_j; the top tenth by q.k are positives with labels falling
// linearly from 20 to 1, the rest negatives with label -1.
//
// Labels: one workgroup per query computes its scores (fp32; 16 lanes per
// key, so each load instruction reads whole 256-byte key rows), selects the
// positives by a radix select on order-preserving score keys and ranks only
// them (score descending, index ascending) with a bitonic sort in LDS.  Step: the
// gradient by the chain rule through h (dh/dz = (1 - h^2)/2), with the pair
// sums as tiled fp32 GEMMs:
//   dL/dHq = 2 eps (rowsum(S) Hq - S Hk)
//   dL/dHk = 2 eps (colsum(S) Hk - S^T Hq) + 2 eta M^T (M Hk),  M_ji = [i <= p_j]
//   dL/dW  = sigma (Q^T dZq + K^T dZk) + 2 lam W A / ||A||_F,   A = W^T W - I
// then W <- W - lr dL/dW.  The loss terms come from the same products.  The
// causal-mask products are sums, not GEMMs: row j of M Hk is the sum of the
// key rows 0..p_j, and row i of M^T (M Hk) the sum of the rows j of M Hk with
// p_j >= i; both are formed from 64-row chunk sums in O((n + J) r) adds.
#include <algorithm>

#include "hata_device.hpp"
#include "hata_launch.hpp"

namespace hata {

namespace {

// ------------------------------------------------------------ labels
constexpr int kLabNT = 256;

// Order-preserving key of a finite fp32 score: a larger score gives a larger
// key, and -0 and +0 (equal scores) give the same key.
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Candidate slots for the ranked positives: a power of two >= the largest
// positive count at this n.
__host__ __device__ inline int label_cand_slots(int n, int pos_permille) {
  const int pp = (n * pos_permille + 999) / 1000;
  const int pmax = pp > 1 ? pp : 1;
  int c = 1;
  while (c < pmax) c <<= 1;
  return c;
}

// One workgroup per query j.  LDS: key[n] (score keys, then the row's
// labels), ck[CL] / ci[CL] (candidate keys and key indices), hist[256],
// misc[16].
//  1. scores of keys 0..p (fp32; 16 lanes per key, lane c multiplying
//     channels 8c .. 8c + 7 from one 16-byte load, the group's 16 partials
//     summed in a fixed order), stored as order-preserving keys;
//  2. radix select, 8 bits per pass from the top: the P-th largest key T and
//     the number `need` of keys equal to T that are positives (ties go to
//     the lower key index, so the first `need` of them in index order);
//  3. the P positives collected by an ordered block scan over runs of
//     consecutive indices, then ranked by a bitonic sort (key descending,
//     index ascending) over the next power of two;
//  4. labels built in LDS and written once per key.
__global__ __launch_bounds__(kLabNT) void labels_kernel(const uint16_t* __restrict__ q,
                                                        const uint16_t* __restrict__ k,
                                                        const int32_t* __restrict__ q_pos, int n,
                                                        int pos_permille, float s_max, float s_min,
                                                        float* __restrict__ S) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int CL = label_cand_slots(n, pos_permille);
  uint32_t* key = reinterpret_cast<uint32_t*>(smem);        // [n]
  uint32_t* ck = key + (n + 3) / 4 * 4;                     // [CL]
  int* ci = reinterpret_cast<int*>(ck + CL);                // [CL]
  uint32_t* hist = reinterpret_cast<uint32_t*>(ci + CL);    // [256]
  uint32_t* misc = hist + 256;                              // [16]
  const int t = threadIdx.x, j = blockIdx.x;
  const int p = min(max(q_pos[j], 0), n - 1);
  const int m = p + 1;
  const int P = max(1, (m * pos_permille + 999) / 1000);

  // 1. scores, four rounds of 16 keys' loads in flight
  {
    const int sub = t & 15, grp = t >> 4;
    float qv[8];
    {
      const uint4 v = *reinterpret_cast<const uint4*>(q + (int64_t)j * kD + 8 * sub);
      const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qv[2 * e] = bf16_lo(w4[e]);
        qv[2 * e + 1] = bf16_hi(w4[e]);
      }
    }
    constexpr int kPerRound = kLabNT / 16, kDepth = 4;
    for (int i0 = 0; i0 < m; i0 += kPerRound * kDepth) {
      uint4 v[kDepth];
#pragma unroll
      for (int u = 0; u < kDepth; ++u) {
        const int i = min(i0 + u * kPerRound + grp, m - 1);
        v[u] = *reinterpret_cast<const uint4*>(k + (int64_t)i * kD + 8 * sub);
      }
#pragma unroll
      for (int u = 0; u < kDepth; ++u) {
        const uint32_t w4[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
        float a = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a = fmaf(qv[2 * e], bf16_lo(w4[e]), a);
          a = fmaf(qv[2 * e + 1], bf16_hi(w4[e]), a);
        }
        a = sum16(a);
        const int i = i0 + u * kPerRound + grp;
        if (sub == 0 && i < m) key[i] = score_key(a);
      }
    }
  }
  __syncthreads();

  // 2. radix select of the P-th largest key (the keys matching `prefix` on
  // the bits decided so far always number at least `need`)
  uint32_t prefix = 0, pmask = 0, need = (uint32_t)P;
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[t] = 0;
    __syncthreads();
    for (int i = t; i < m; i += kLabNT) {
      const uint32_t u = key[i];
      if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
    }
    __syncthreads();
    const uint32_t c = hist[255 - t];  // thread t: digit 255 - t, counted from the top
    uint32_t tot;
    const uint32_t above = block_excl_scan_u32(c, misc, &tot);
    if (above < need && above + c >= need) {
      misc[8] = 255u - (uint32_t)t;
      misc[9] = need - above;
    }
    __syncthreads();
    prefix |= misc[8] << shift;
    pmask |= 255u << shift;
    need = misc[9];
    __syncthreads();
  }
  const uint32_t T = prefix;

  // 3. collect: every key above T, and the first `need` keys equal to T in
  // index order; thread t owns indices [t R, t R + R)
  {
    const int R = (m + kLabNT - 1) / kLabNT;
    const int i0 = t * R, i1 = min(i0 + R, m);
    uint32_t ngt = 0, neq = 0;
    for (int i = i0; i < i1; ++i) {
      const uint32_t u = key[i];
      ngt += u > T ? 1u : 0u;
      neq += u == T ? 1u : 0u;
    }
    uint32_t tot;
    const uint32_t pre = block_excl_scan_u32(ngt | (neq << 16), misc, &tot);  // m <= 8192
    uint32_t gpos = pre & 0xFFFFu, epos = pre >> 16;
    const uint32_t cgt = (uint32_t)P - need;  // keys above T
    for (int i = i0; i < i1; ++i) {
      const uint32_t u = key[i];
      if (u > T) {
        ck[gpos] = u;
        ci[gpos] = i;
        ++gpos;
      } else if (u == T) {
        if (epos < need) {
          ck[cgt + epos] = u;
          ci[cgt + epos] = i;
        }
        ++epos;
      }
    }
  }
  int Lc = 1;
  while (Lc < P) Lc <<= 1;
  for (int r = P + t; r < Lc; r += kLabNT) {  // padding ranks last
    ck[r] = 0u;
    ci[r] = 0x7FFFFFFF;
  }
  __syncthreads();
  for (int sz = 2; sz <= Lc; sz <<= 1) {
    for (int st = sz >> 1; st > 0; st >>= 1) {
      for (int e = t; e < Lc / 2; e += kLabNT) {
        const int lo = 2 * e - (e & (st - 1));
        const int hi = lo + st;
        const bool up = (lo & sz) == 0;  // this half sorts "first" to the front
        const uint32_t ka = ck[lo], kb = ck[hi];
        const int ia = ci[lo], ib = ci[hi];
        const bool b_first = (kb > ka) || (kb == ka && ib < ia);
        if (b_first == up) {
          ck[lo] = kb; ck[hi] = ka;
          ci[lo] = ib; ci[hi] = ia;
        }
      }
      __syncthreads();
    }
  }

  // 4. labels: -1 for keys 0..p, then the ranked positives
  float* lab = reinterpret_cast<float*>(key);
  for (int i = t; i < m; i += kLabNT) lab[i] = -1.f;
  __syncthreads();
  for (int r = t; r < P; r += kLabNT)
    lab[ci[r]] = (P == 1) ? s_max : s_max - (s_max - s_min) * (float)r / (float)(P - 1);
  __syncthreads();
  float* row = S + (int64_t)j * n;
  for (int i = t; i < n; i += kLabNT) row[i] = i < m ? lab[i] : 0.f;
}

// ------------------------------------------------------------ tiled GEMM
// C[M][N] = alpha * sum_k A(m, k) B(k, n) (+ C if accumulate), fp32.  A and
// B are read through accessor structs; kColFast says whether consecutive
// column indices are adjacent in memory, and the tile fill lets consecutive
// lanes walk that index so the global reads coalesce.  64 x 64 output tiles,
// 32-deep k steps staged in LDS (rows padded by 4 floats: 16-byte aligned
// vector reads, conflict-free column writes), the next step's operands held
// in registers while the current one is multiplied.  The 4 waves take the
// tile's 32 x 32 quarters on v_mfma_f32_32x32x2_f32 (fp32 operands and
// accumulation): per MFMA, lane l brings A(row l % 32, k 2 kk + l / 32) and
// B(k 2 kk + l / 32, col l % 32).  Products with few output tiles and a
// long k split k over blockIdx.z; each split writes its own partial tile and
// a second kernel adds the partials in split order (deterministic).
// Each accessor also reads kVec consecutive elements along its contiguous
// index with one 16-byte load (vec), allowed when ld is a multiple of kVec
// (the base pointers are 16-byte aligned).
struct AccF32 {  // row-major [rows][ld]
  static constexpr bool kColFast = true;
  static constexpr int kVec = 4;
  const float* p; int ld;
  __device__ float operator()(int r, int c) const { return p[(int64_t)r * ld + c]; }
  __device__ void vec(int r, int c, float* o) const {  // (r, c .. c + 3)
    const float4 v = *reinterpret_cast<const float4*>(p + (int64_t)r * ld + c);
    o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
  }
  __device__ bool vec_ok() const { return (ld & 3) == 0; }
};
struct AccF32T {  // element (r, c) of the transpose of a row-major [.][ld]
  static constexpr bool kColFast = false;
  static constexpr int kVec = 4;
  const float* p; int ld;
  __device__ float operator()(int r, int c) const { return p[(int64_t)c * ld + r]; }
  __device__ void vec(int r, int c, float* o) const {  // (r .. r + 3, c)
    const float4 v = *reinterpret_cast<const float4*>(p + (int64_t)c * ld + r);
    o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
  }
  __device__ bool vec_ok() const { return (ld & 3) == 0; }
};
struct AccBf16 {
  static constexpr bool kColFast = true;
  static constexpr int kVec = 8;
  const uint16_t* p; int ld;
  __device__ float operator()(int r, int c) const { return __uint_as_float((uint32_t)p[(int64_t)r * ld + c] << 16); }
  __device__ void vec(int r, int c, float* o) const {  // (r, c .. c + 7)
    const uint4 v = *reinterpret_cast<const uint4*>(p + (int64_t)r * ld + c);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) { o[2 * i] = bf16_lo(w[i]); o[2 * i + 1] = bf16_hi(w[i]); }
  }
  __device__ bool vec_ok() const { return (ld & 7) == 0; }
};
struct AccBf16T {
  static constexpr bool kColFast = false;
  static constexpr int kVec = 8;
  const uint16_t* p; int ld;
  __device__ float operator()(int r, int c) const { return __uint_as_float((uint32_t)p[(int64_t)c * ld + r] << 16); }
  __device__ void vec(int r, int c, float* o) const {  // (r .. r + 7, c)
    const uint4 v = *reinterpret_cast<const uint4*>(p + (int64_t)c * ld + r);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) { o[2 * i] = bf16_lo(w[i]); o[2 * i + 1] = bf16_hi(w[i]); }
  }
  __device__ bool vec_ok() const { return (ld & 7) == 0; }
};
struct AccGramMinusI {  // (W^T W - I)[r][c] from a precomputed W^T W
  static constexpr bool kColFast = true;
  static constexpr int kVec = 4;
  const float* p; int ld;
  __device__ float operator()(int r, int c) const { return p[(int64_t)r * ld + c] - (r == c ? 1.f : 0.f); }
  __device__ void vec(int r, int c, float* o) const {
    const float4 v = *reinterpret_cast<const float4*>(p + (int64_t)r * ld + c);
    o[0] = v.x - (r == c ? 1.f : 0.f); o[1] = v.y - (r == c + 1 ? 1.f : 0.f);
    o[2] = v.z - (r == c + 2 ? 1.f : 0.f); o[3] = v.w - (r == c + 3 ? 1.f : 0.f);
  }
  __device__ bool vec_ok() const { return (ld & 3) == 0; }
};

constexpr int kT = 64, kKS = 32, kLdsRow = kT + 4, kFill = kT * kKS / 256;

// Tile fills in 16-byte pieces: piece q of the A tile (rows m0 .., k k0 ..)
// or of the B tile (k k0 .., columns n0 ..) covers V = Acc::kVec consecutive
// elements along the accessor's contiguous index, consecutive pieces walking
// that index so a wave's loads coalesce.  (mm, kk) / (kk, nn) is the first
// element; the others follow along k (dk = 1) or along m / n.
template <class Acc>
__device__ inline void a_piece(int q, int& mm, int& kk) {
  constexpr int V = Acc::kVec;
  if constexpr (Acc::kColFast) { mm = q / (kKS / V); kk = (q % (kKS / V)) * V; }
  else { kk = q / (kT / V); mm = (q % (kT / V)) * V; }
}
template <class Acc>
__device__ inline void b_piece(int q, int& kk, int& nn) {
  constexpr int V = Acc::kVec;
  if constexpr (Acc::kColFast) { kk = q / (kT / V); nn = (q % (kT / V)) * V; }
  else { nn = q / (kKS / V); kk = (q % (kKS / V)) * V; }
}

template <class A, class B>
__global__ __launch_bounds__(256) void gemm_kernel(int M, int N, int K, int kchunk, A a, B b,
                                                   float* __restrict__ C, int ldc, float alpha, int accumulate,
                                                   float* __restrict__ part, int tanh_out) {
  __shared__ __align__(16) float as[kKS][kLdsRow];
  __shared__ __align__(16) float bs[kKS][kLdsRow];
  const int t = threadIdx.x;
  const int m0 = blockIdx.y * kT, n0 = blockIdx.x * kT;
  const int kbeg = blockIdx.z * kchunk, kend = min(K, kbeg + kchunk);
  // this thread's pieces: A::kVec (B::kVec) elements each, kFill in all
  constexpr int PA = kFill / A::kVec, PB = kFill / B::kVec;
  float ra[kFill], rb[kFill];
  const bool va = a.vec_ok(), vb = b.vec_ok();
  auto fetch = [&](int k0) {
#pragma unroll
    for (int u = 0; u < PA; ++u) {
      int mm, kk;
      a_piece<A>(t + 256 * u, mm, kk);
      float* o = ra + u * A::kVec;
      const int m = m0 + mm, k = k0 + kk;
      // the piece's last element (along k or along m)
      const bool full = A::kColFast ? (m < M && k + A::kVec <= kend) : (m + A::kVec <= M && k < kend);
      if (va && full) {
        a.vec(m, k, o);
      } else {
#pragma unroll
        for (int i = 0; i < A::kVec; ++i) {
          const int mi = A::kColFast ? m : m + i, ki = A::kColFast ? k + i : k;
          o[i] = (mi < M && ki < kend) ? a(mi, ki) : 0.f;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < PB; ++u) {
      int kk, nn;
      b_piece<B>(t + 256 * u, kk, nn);
      float* o = rb + u * B::kVec;
      const int k = k0 + kk, n = n0 + nn;
      const bool full = B::kColFast ? (k < kend && n + B::kVec <= N) : (k + B::kVec <= kend && n < N);
      if (vb && full) {
        b.vec(k, n, o);
      } else {
#pragma unroll
        for (int i = 0; i < B::kVec; ++i) {
          const int ki = B::kColFast ? k : k + i, ni = B::kColFast ? n + i : n;
          o[i] = (ki < kend && ni < N) ? b(ki, ni) : 0.f;
        }
      }
    }
  };
  typedef float f32x16 __attribute__((ext_vector_type(16)));
  const int lane = t & 63, wv = t >> 6, wm = wv >> 1, wn = wv & 1;
  f32x16 acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  if (kbeg < kend) fetch(kbeg);
  for (int k0 = kbeg; k0 < kend; k0 += kKS) {
#pragma unroll
    for (int u = 0; u < PA; ++u) {
      int mm, kk;
      a_piece<A>(t + 256 * u, mm, kk);
#pragma unroll
      for (int i = 0; i < A::kVec; ++i) {
        if constexpr (A::kColFast) as[kk + i][mm] = ra[u * A::kVec + i];
        else as[kk][mm + i] = ra[u * A::kVec + i];
      }
    }
#pragma unroll
    for (int u = 0; u < PB; ++u) {
      int kk, nn;
      b_piece<B>(t + 256 * u, kk, nn);
#pragma unroll
      for (int i = 0; i < B::kVec; ++i) {
        if constexpr (B::kColFast) bs[kk][nn + i] = rb[u * B::kVec + i];
        else bs[kk + i][nn] = rb[u * B::kVec + i];
      }
    }
    __syncthreads();
    if (k0 + kKS < kend) fetch(k0 + kKS);
#pragma unroll
    for (int kk = 0; kk < kKS / 2; ++kk) {
      const float av = as[2 * kk + (lane >> 5)][32 * wm + (lane & 31)];
      const float bv = bs[2 * kk + (lane >> 5)][32 * wn + (lane & 31)];
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc, 0, 0, 0);
    }
    __syncthreads();
  }
  // accumulator i: row 8 (i / 4) + i % 4 + 4 (lane / 32), column lane % 32
  // of this wave's quarter
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int mm = m0 + 32 * wm + 8 * (i >> 2) + (i & 3) + 4 * (lane >> 5);
    const int nn = n0 + 32 * wn + (lane & 31);
    const float accv = acc[i];
    if (mm < M && nn < N) {
      if (part) {
        part[((int64_t)blockIdx.z * M + mm) * N + nn] = accv;
      } else {
        float* c = C + (int64_t)mm * ldc + nn;
        const float v = alpha * accv + (accumulate ? *c : 0.f);
        *c = tanh_out ? tanhf(v) : v;
      }
    }
  }
}

// C = alpha * sum_z part[z] (+ C), splits added in order; four adjacent
// outputs per thread (N and ldc are multiples of 4), eight splits' loads
// issued before their adds
__global__ void splitk_reduce_kernel(const float* __restrict__ part, int splits, int M, int N,
                                     float* __restrict__ C, int ldc, float alpha, int accumulate) {
  const int64_t e4 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t mn = (int64_t)M * N;
  if (e4 * 4 >= mn) return;
  const float4* p4 = reinterpret_cast<const float4*>(part) + e4;
  const int64_t zs = mn / 4;
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  int z = 0;
  for (; z + 8 <= splits; z += 8) {
    float4 t[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) t[u] = p4[(z + u) * zs];
#pragma unroll
    for (int u = 0; u < 8; ++u) { v.x += t[u].x; v.y += t[u].y; v.z += t[u].z; v.w += t[u].w; }
  }
  for (; z < splits; ++z) {
    const float4 t = p4[z * zs];
    v.x += t.x; v.y += t.y; v.z += t.z; v.w += t.w;
  }
  const int64_t e = e4 * 4;
  float* c = C + (e / N) * ldc + e % N;
  const float o[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int u = 0; u < 4; ++u) c[u] = alpha * o[u] + (accumulate ? c[u] : 0.f);
}

}  // namespace

// number of k splits for an M x N x K product: aim at about four
// workgroups per compute unit, each split at least 128 deep, or one k step
// (32) deep for products of k <= 512 (W^T W, W A, Q^T dZq: few output
// tiles, so otherwise a handful of workgroups would walk k alone)
int train_gemm_splits(int M, int N, int K) {
  const int tiles = ((M + kT - 1) / kT) * ((N + kT - 1) / kT);
  const int want = (1024 + tiles - 1) / tiles;
  const int s = std::min(want, K / (K <= 512 ? kKS : 128));
  return std::max(s, 1);
}

namespace {

template <class A, class B>
hipError_t gemm(int M, int N, int K, A a, B b, float* C, int ldc, float alpha, bool accumulate, float* part,
                hipStream_t s, bool tanh_out = false) {
  const int splits = tanh_out ? 1 : train_gemm_splits(M, N, K);
  const int kchunk = splits == 1 ? K : ((K + splits - 1) / splits + kKS - 1) / kKS * kKS;
  const int z = splits == 1 ? 1 : (K + kchunk - 1) / kchunk;
  dim3 grid((unsigned)((N + kT - 1) / kT), (unsigned)((M + kT - 1) / kT), (unsigned)z);
  hipLaunchKernelGGL((gemm_kernel<A, B>), grid, dim3(256), 0, s, M, N, K, kchunk, a, b, C, ldc, alpha,
                     accumulate ? 1 : 0, z == 1 ? (float*)nullptr : part, tanh_out ? 1 : 0);
  if (z > 1) {
    if (N % 4 != 0 || ldc % 4 != 0) return hipErrorInvalidValue;
    const int64_t cnt = (int64_t)M * N / 4;
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((cnt + 255) / 256)), dim3(256), 0, s, part, z, M, N,
                       C, ldc, alpha, accumulate ? 1 : 0);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------ causal-mask sums
// M_ji = [i <= p_j] with p_j clamped into [0, n - 1].  Fixed summation
// orders throughout (no atomics), so the results do not vary between runs.
constexpr int kMaskRows = 64;  // key rows per chunk

// The kernels below are bound by the latency of their loads, so every loop
// over rows or queries loads all its operands first (indices clamped into
// range, a select dropping the extra ones) and adds them afterwards.

// T[c][col] = sum of Hk rows 64c .. 64c + 63.  Workgroup = (chunk, 64
// columns), thread = (column, quarter u): rows 16u .. 16u + 15 ascending,
// then the four sums in quarter order.
__global__ __launch_bounds__(256) void mask_chunk_sums_kernel(const float* __restrict__ Hk, int n, int r,
                                                              float* __restrict__ T) {
  __shared__ float qs[4][64];
  const int t = threadIdx.x, lane = t & 63, u = t >> 6;
  const int c = blockIdx.x;
  const int col = blockIdx.y * 64 + lane;
  const int cc = min(col, r - 1);
  const int i0 = c * kMaskRows + 16 * u, i1 = min(n, c * kMaskRows + kMaskRows);
  float v[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) v[q] = Hk[(int64_t)min(i0 + q, n - 1) * r + cc];
  float s = 0.f;
#pragma unroll
  for (int q = 0; q < 16; ++q) s += (i0 + q < i1) ? v[q] : 0.f;
  qs[u][lane] = s;
  __syncthreads();
  if (u == 0 && col < r) T[(int64_t)c * r + col] = ((qs[0][lane] + qs[1][lane]) + qs[2][lane]) + qs[3][lane];
}

// Cm[j] = (M Hk)_j = sum_{i <= p_j} Hk[i].  Workgroup = (query j, 64
// columns), thread = (column, quarter u): quarter u sums the chunk sums
// u, u + 4, ... before p_j's chunk (32 loads in flight at a time), then rows
// 16u .. 16u + 15 of that chunk up to p_j (ascending); the four sums are
// added in quarter order.
__global__ __launch_bounds__(256) void mask_rows_kernel(const float* __restrict__ Hk, const float* __restrict__ T,
                                                        const int32_t* __restrict__ pos, int J, int n, int r,
                                                        float* __restrict__ Cm) {
  __shared__ float qs[4][64];
  const int t = threadIdx.x, lane = t & 63, u = t >> 6;
  const int j = blockIdx.x;
  const int col = blockIdx.y * 64 + lane;
  const int cc = min(col, r - 1);
  const int p = min(max(pos[j], 0), n - 1);
  const int cj = p / kMaskRows;
  float s = 0.f;
  for (int c0 = u; c0 < cj; c0 += 4 * 32) {
    float v[32];
#pragma unroll
    for (int q = 0; q < 32; ++q) v[q] = T[(int64_t)min(c0 + 4 * q, cj - 1) * r + cc];
#pragma unroll
    for (int q = 0; q < 32; ++q) s += (c0 + 4 * q < cj) ? v[q] : 0.f;
  }
  const int ib = cj * kMaskRows + 16 * u;
  float v[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) v[q] = Hk[(int64_t)min(ib + q, n - 1) * r + cc];
#pragma unroll
  for (int q = 0; q < 16; ++q) s += (ib + q <= p) ? v[q] : 0.f;
  qs[u][lane] = s;
  __syncthreads();
  if (u == 0 && col < r) Cm[(int64_t)j * r + col] = ((qs[0][lane] + qs[1][lane]) + qs[2][lane]) + qs[3][lane];
}

// MtC[i] = (M^T Cm)_i = sum_{j : p_j >= i} Cm[j].  Workgroup = (64-row chunk,
// 64 columns), thread = (column, quarter u).  Queries are taken in batches of
// 256: those positioned past the chunk add to every row of it (quarter u
// sums batch entries 64u .. 64u + 63 in order; the four sums are added in
// quarter order at the end); those inside the chunk are listed in LDS in
// query order and added, 8 list entries per round of loads, to the rows at
// or before their position (quarter u owns rows 16u .. 16u + 15).
__global__ __launch_bounds__(256) void mask_cols_kernel(const float* __restrict__ Cm, const int32_t* __restrict__ pos,
                                                        int J, int n, int r, float* __restrict__ MtC) {
  __shared__ int bp[256];           // positions of the batch (-1 past J)
  __shared__ int lj[256], lp[256];  // in-chunk queries of the batch, in query order
  __shared__ int wcnt[4];
  __shared__ float qs[4][64];
  const int t = threadIdx.x, lane = t & 63, u = t >> 6;
  const int col = blockIdx.y * 64 + lane;
  const int cc = min(col, r - 1);
  const int i0 = blockIdx.x * kMaskRows, i1 = min(n, i0 + kMaskRows);
  const int r0 = i0 + 16 * u;  // this thread's first row
  float past = 0.f;
  float acc[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) acc[q] = 0.f;
  for (int jb = 0; jb < J; jb += 256) {
    const int j = jb + t;
    const int p = (j < J) ? min(max(pos[j], 0), n - 1) : -1;
    bp[t] = p;
    const bool in = p >= i0 && p < i1;
    const uint64_t m = __ballot(in);
    if (lane == 0) wcnt[u] = __popcll(m);
    __syncthreads();
    int off = 0;
    for (int w = 0; w < u; ++w) off += wcnt[w];
    const int nin = wcnt[0] + wcnt[1] + wcnt[2] + wcnt[3];
    if (in) {
      const int e = off + __popcll(m & ((1ull << lane) - 1));
      lj[e] = j;
      lp[e] = p;
    }
    __syncthreads();
    {
      float v[64];
#pragma unroll
      for (int e = 0; e < 64; ++e) v[e] = Cm[(int64_t)min(jb + 64 * u + e, J - 1) * r + cc];
#pragma unroll
      for (int e = 0; e < 64; ++e) past += (bp[64 * u + e] >= i1) ? v[e] : 0.f;
    }
    for (int e0 = 0; e0 < nin; e0 += 8) {
      float v[8];
      int pe[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int e = min(e0 + q, nin - 1);
        v[q] = Cm[(int64_t)lj[e] * r + cc];
        pe[q] = (e0 + q < nin) ? lp[e] : -1;
      }
#pragma unroll
      for (int q = 0; q < 8; ++q)
#pragma unroll
        for (int x = 0; x < 16; ++x)
          if (pe[q] >= r0 + x) acc[x] += v[q];
    }
    __syncthreads();
  }
  qs[u][lane] = past;
  __syncthreads();
  const float tot = ((qs[0][lane] + qs[1][lane]) + qs[2][lane]) + qs[3][lane];
  if (col < r) {
#pragma unroll
    for (int q = 0; q < 16; ++q)
      if (r0 + q < i1) MtC[(int64_t)(r0 + q) * r + col] = tot + acc[q];
  }
}

// ------------------------------------------------------------ elementwise
// rows of X [rows][cols]: out[r] = sum_c X[r][c] (sums S_j) or columns
__global__ void row_sums_kernel(const float* __restrict__ X, int rows, int cols, float* __restrict__ out) {
  const int r = blockIdx.x;
  const float* x = X + (int64_t)r * cols;
  // eight running sums per thread (columns c + 256 u), so eight loads are in
  // flight; added in a fixed order
  float a8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int c = threadIdx.x;
  for (; c + 7 * 256 < cols; c += 8 * 256) {
#pragma unroll
    for (int u = 0; u < 8; ++u) a8[u] += x[c + 256 * u];
  }
  for (; c < cols; c += 256) a8[0] += x[c];
  const float a = ((a8[0] + a8[1]) + (a8[2] + a8[3])) + ((a8[4] + a8[5]) + (a8[6] + a8[7]));
  __shared__ float red[256];
  red[threadIdx.x] = a;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[r] = red[0];
}
// column sums in two passes: pass 1 gives kColChunks partial sums per
// column (workgroup = 64 columns x 4 row slices of one row chunk), pass 2
// adds the partials in chunk order
constexpr int kColChunks = 16;
__global__ void col_sums_part_kernel(const float* __restrict__ X, int rows, int cols, float* __restrict__ part) {
  __shared__ float red[4][64];
  const int c = blockIdx.x * 64 + (threadIdx.x & 63), sl = threadIdx.x >> 6;
  const int per = (rows + kColChunks - 1) / kColChunks;
  const int r0 = blockIdx.y * per, r1 = min(rows, r0 + per);
  float a = 0.f;
  if (c < cols)
    for (int r = r0 + sl; r < r1; r += 4) a += X[(int64_t)r * cols + c];
  red[sl][threadIdx.x & 63] = a;
  __syncthreads();
  if (sl == 0 && c < cols) {
    const int l = threadIdx.x;
    part[(int64_t)blockIdx.y * cols + c] = ((red[0][l] + red[1][l]) + red[2][l]) + red[3][l];
  }
}
__global__ void col_sums_finish_kernel(const float* __restrict__ part, int cols, float* __restrict__ out) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= cols) return;
  float a = 0.f;
#pragma unroll
  for (int z = 0; z < kColChunks; ++z) a += part[(int64_t)z * cols + c];
  out[c] = a;
}

// dZ = (2 eps (rs * H - P) + 2 eta Qb) * (1 - H^2) / 2 per element, where P
// is the pair product (S Hk or S^T Hq) and Qb the balance product (M^T C,
// or null for the queries).  Also the per-row partial loss sums:
// part[3 row] = rs * ||H_row||^2 (for the similarity term),
// part[3 row + 1] = H_row . P_row and part[3 row + 2] = ||Cb_row||^2 (the
// balance term; Cb = M Hk for the queries, null for the keys).
__global__ __launch_bounds__(256) void dz_kernel(const float* __restrict__ H, const float* __restrict__ P,
                                                 const float* __restrict__ Qb, const float* __restrict__ Cb,
                                                 const float* __restrict__ rs, int rows, int r, float eps, float eta,
                                                 float* __restrict__ dZ, float* __restrict__ part) {
  // one wave per row (four rows per workgroup); the row's partial sums are
  // added per lane in column order, then over the wave in a fixed order
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;  // the whole wave
  float a1 = 0.f, a2 = 0.f, a3 = 0.f;
  const float w = rs[row];
  for (int c = lane; c < r; c += 64) {
    const int64_t e = (int64_t)row * r + c;
    const float h = H[e], pp = P[e];
    float g = 2.f * eps * (w * h - pp);
    if (Qb) g += 2.f * eta * Qb[e];
    dZ[e] = g * (1.f - h * h) * 0.5f;
    a1 += w * h * h;
    a2 += h * pp;
    if (Cb) a3 += Cb[e] * Cb[e];
  }
  auto wave_sum = [](float v) {
    const int s16 = __float_as_int(sum16(v));  // each group of 16 lanes holds its sum
    return ((__int_as_float(__builtin_amdgcn_readlane(s16, 0)) + __int_as_float(__builtin_amdgcn_readlane(s16, 16))) +
            __int_as_float(__builtin_amdgcn_readlane(s16, 32))) +
           __int_as_float(__builtin_amdgcn_readlane(s16, 48));
  };
  a1 = wave_sum(a1);
  a2 = wave_sum(a2);
  a3 = wave_sum(a3);
  if (lane == 0) {
    part[3 * row] = a1;
    part[3 * row + 1] = a2;
    part[3 * row + 2] = a3;
  }
}

// Final loss terms and the decorrelation factor, one workgroup of 1024
// threads (fixed order): loss[0..3] = total, similarity, balance,
// decorrelation; fac[0] = 2 lam / ||A||_F (0 when A == 0), A = W^T W - I.
constexpr int kLossNT = 1024;
__global__ __launch_bounds__(kLossNT) void loss_kernel(const float* __restrict__ part_q, int J,
                                                       const float* __restrict__ part_k, int n, int r,
                                                       const float* __restrict__ gram, float eps, float eta,
                                                       float lam, float* __restrict__ loss,
                                                       float* __restrict__ fac) {
  __shared__ float red[4][kLossNT];
  const int t = threadIdx.x;
  float sq = 0.f, sk = 0.f, bal = 0.f, dec = 0.f;
  for (int j = t; j < J; j += kLossNT) {
    sq += part_q[3 * j] - 2.f * part_q[3 * j + 1];
    bal += part_q[3 * j + 2];
  }
#pragma unroll 4
  for (int i = t; i < n; i += kLossNT) sk += part_k[3 * i];
#pragma unroll 4
  for (int e = t; e < r * r; e += kLossNT) {
    const float v = gram[e] - ((e / r) == (e % r) ? 1.f : 0.f);
    dec += v * v;
  }
  red[0][t] = sq; red[1][t] = sk; red[2][t] = bal; red[3][t] = dec;
  __syncthreads();
  for (int o = kLossNT / 2; o > 0; o >>= 1) {
    if (t < o)
      for (int q = 0; q < 4; ++q) red[q][t] += red[q][t + o];
    __syncthreads();
  }
  if (t == 0) {
    const float sim = eps * (red[0][0] + red[1][0]);
    const float b = eta * red[2][0];
    const float na = sqrtf(red[3][0]);
    const float d = lam * na;
    loss[0] = sim + b + d; loss[1] = sim; loss[2] = b; loss[3] = d;
    fac[0] = na > 0.f ? 2.f * lam / na : 0.f;
  }
}

// g = dW + fac * W A (the full gradient), W <- W - lr g; optional gradient copy
__global__ void update_kernel(float* __restrict__ W, const float* __restrict__ dW, const float* __restrict__ WA,
                              const float* __restrict__ fac, float* __restrict__ grad, int count, float lr) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= count) return;
  const float g = dW[i] + fac[0] * WA[i];
  if (grad) grad[i] = g;
  W[i] = fmaf(-lr, g, W[i]);  // one rounding of the updated weight
}

}  // namespace

size_t label_lds_bytes(int n, int pos_permille) {
  return ((size_t)(n + 3) / 4 * 4 + 2 * (size_t)label_cand_slots(n, pos_permille) + 256 + 16) * 4;
}

hipError_t launch_hash_labels(const uint16_t* q, const uint16_t* k, const int32_t* q_pos, int J, int n,
                              int pos_permille, float s_max, float s_min, float* S, hipStream_t s) {
  static bool configured = false;
  const size_t lds = label_lds_bytes(n, pos_permille);
  if (!configured) {  // the largest size any call can need
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&labels_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)label_lds_bytes(kMaxLabelKeys, 1000));
    if (e != hipSuccess) return e;
    configured = true;
  }
  hipLaunchKernelGGL(labels_kernel, dim3(J), dim3(kLabNT), lds, s, q, k, q_pos, n, pos_permille, s_max, s_min, S);
  return hipGetLastError();
}

TrainPlan plan_train(int J, int n, int r) {
  TrainPlan p;
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  size_t off = 0;
  auto take = [&](size_t floats) { const size_t o = off; off = al(off + floats * 4); return o; };
  p.hq = take((size_t)J * r);
  p.hk = take((size_t)n * r);
  p.shk = take((size_t)J * r);
  p.sthq = take((size_t)n * r);
  p.cm = take((size_t)J * r);
  p.mtc = take((size_t)n * r);
  p.rs = take((size_t)J);
  p.cs = take((size_t)n);
  p.dzq = take((size_t)J * r);
  p.dzk = take((size_t)n * r);
  p.gram = take((size_t)r * r);
  p.dw = take((size_t)kD * r);
  p.wa = take((size_t)kD * r);
  p.partq = take((size_t)3 * J);
  p.partk = take((size_t)3 * n);
  p.fac = take(4);
  // the largest split-k partial buffer over the step's products
  const int shapes[8][3] = {{J, r, kD}, {n, r, kD}, {J, r, n}, {n, r, J},
                            {kD, r, J}, {kD, r, n}, {r, r, kD}, {kD, r, r}};
  size_t part = 0;
  for (const auto& g : shapes) {
    const int sp = train_gemm_splits(g[0], g[1], g[2]);
    if (sp > 1) part = std::max(part, (size_t)sp * g[0] * g[1]);
  }
  part = std::max(part, (size_t)kColChunks * n);  // column-sum partials
  part = std::max(part, (size_t)((n + kMaskRows - 1) / kMaskRows) * r);  // chunk sums of Hk
  p.part = take(part);
  p.total = off;
  return p;
}

hipError_t launch_hash_train_step(const TrainPlan& p, const uint16_t* q, const uint16_t* k, const int32_t* q_pos,
                                  const float* S, int J, int n, int r, float sigma, float eps, float eta,
                                  float lam, float lr, float* W, float* grad, float* loss, unsigned char* ws,
                                  hipStream_t s) {
  auto F = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
  float *Hq = F(p.hq), *Hk = F(p.hk), *SHk = F(p.shk), *StHq = F(p.sthq), *Cm = F(p.cm), *MtC = F(p.mtc);
  float *rs = F(p.rs), *cs = F(p.cs), *dZq = F(p.dzq), *dZk = F(p.dzk), *gram = F(p.gram), *dW = F(p.dw);
  float *WA = F(p.wa), *partq = F(p.partq), *partk = F(p.partk), *fac = F(p.fac), *part = F(p.part);
  hipError_t e;
#define HATA_TRY(x) do { e = (x); if (e != hipSuccess) return e; } while (0)
  // H = tanh(sigma/2 * X W)
  HATA_TRY(gemm(J, r, kD, AccBf16{q, kD}, AccF32{W, r}, Hq, r, 0.5f * sigma, false, part, s, true));
  HATA_TRY(gemm(n, r, kD, AccBf16{k, kD}, AccF32{W, r}, Hk, r, 0.5f * sigma, false, part, s, true));
  // pair products, label sums, balance products
  HATA_TRY(gemm(J, r, n, AccF32{S, n}, AccF32{Hk, r}, SHk, r, 1.f, false, part, s));
  HATA_TRY(gemm(n, r, J, AccF32T{S, n}, AccF32{Hq, r}, StHq, r, 1.f, false, part, s));
  {
    const unsigned nc = (unsigned)((n + kMaskRows - 1) / kMaskRows), cb = (unsigned)((r + 63) / 64);
    hipLaunchKernelGGL(mask_chunk_sums_kernel, dim3(nc, cb), dim3(256), 0, s, (const float*)Hk, n, r,
                       part);
    hipLaunchKernelGGL(mask_rows_kernel, dim3((unsigned)J, cb), dim3(256), 0, s, (const float*)Hk,
                       (const float*)part, q_pos, J, n, r, Cm);
    hipLaunchKernelGGL(mask_cols_kernel, dim3(nc, cb), dim3(256), 0, s, (const float*)Cm, q_pos, J, n, r, MtC);
    HATA_TRY(hipGetLastError());
  }
  hipLaunchKernelGGL(row_sums_kernel, dim3(J), dim3(256), 0, s, S, J, n, rs);
  hipLaunchKernelGGL(col_sums_part_kernel, dim3((unsigned)((n + 63) / 64), kColChunks), dim3(256), 0, s, S, J, n,
                     part);
  hipLaunchKernelGGL(col_sums_finish_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, part, n, cs);
  HATA_TRY(hipGetLastError());
  // dZ and the per-row loss parts
  hipLaunchKernelGGL(dz_kernel, dim3((unsigned)((J + 3) / 4)), dim3(256), 0, s, Hq, SHk, (const float*)nullptr, (const float*)Cm, rs, J, r,
                     eps, eta, dZq, partq);
  hipLaunchKernelGGL(dz_kernel, dim3((unsigned)((n + 3) / 4)), dim3(256), 0, s, Hk, StHq, (const float*)MtC, (const float*)nullptr, cs, n,
                     r, eps, eta, dZk, partk);
  HATA_TRY(hipGetLastError());
  // dW = sigma (Q^T dZq + K^T dZk)
  HATA_TRY(gemm(kD, r, J, AccBf16T{q, kD}, AccF32{dZq, r}, dW, r, sigma, false, part, s));
  HATA_TRY(gemm(kD, r, n, AccBf16T{k, kD}, AccF32{dZk, r}, dW, r, sigma, true, part, s));
  // decorrelation: gram = W^T W, WA = W (gram - I), dW += 2 lam / ||A|| * WA
  HATA_TRY(gemm(r, r, kD, AccF32T{W, r}, AccF32{W, r}, gram, r, 1.f, false, part, s));
  HATA_TRY(gemm(kD, r, r, AccF32{W, r}, AccGramMinusI{gram, r}, WA, r, 1.f, false, part, s));
  hipLaunchKernelGGL(loss_kernel, dim3(1), dim3(kLossNT), 0, s, partq, J, partk, n, r, gram, eps, eta, lam, loss,
                     fac);
  hipLaunchKernelGGL(update_kernel, dim3((kD * r + 255) / 256), dim3(256), 0, s, W, (const float*)dW,
                     (const float*)WA, (const float*)fac, grad, kD * r, lr);
  return hipGetLastError();
#undef HATA_TRY
}

}  // namespace hata
