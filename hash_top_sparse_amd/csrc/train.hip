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
// Labels: one workgroup per query computes its scores (fp32) and sorts
// (score descending, index ascending) with a bitonic sort in LDS.  Step: the
// gradient by the chain rule through h (dh/dz = (1 - h^2)/2), with the pair
// sums as tiled fp32 GEMMs:
//   dL/dHq = 2 eps (rowsum(S) Hq - S Hk)
//   dL/dHk = 2 eps (colsum(S) Hk - S^T Hq) + 2 eta M^T (M Hk),  M_ji = [i <= p_j]
//   dL/dW  = sigma (Q^T dZq + K^T dZk) + 2 lam W A / ||A||_F,   A = W^T W - I
// then W <- W - lr dL/dW.  The loss terms come from the same products.
#include "hata_device.hpp"
#include "hata_launch.hpp"

namespace hata {

namespace {

// ------------------------------------------------------------ labels
constexpr int kLabNT = 256;

__global__ __launch_bounds__(kLabNT) void labels_kernel(const uint16_t* __restrict__ q,
                                                        const uint16_t* __restrict__ k,
                                                        const int32_t* __restrict__ q_pos, int n,
                                                        int pos_permille, float s_max, float s_min,
                                                        float* __restrict__ S) {
  extern __shared__ __align__(16) unsigned char smem[];
  float* qs = reinterpret_cast<float*>(smem);          // [128]
  float* key = qs + kD;                                 // [L] scores
  int* ids = reinterpret_cast<int*>(key + kMaxLabelKeys);  // [L]
  const int t = threadIdx.x, j = blockIdx.x;
  const int p = min(max(q_pos[j], 0), n - 1);
  const int m = p + 1;
  int L = 1;
  while (L < m) L <<= 1;
  for (int c = t; c < kD; c += kLabNT) qs[c] = __uint_as_float((uint32_t)q[(int64_t)j * kD + c] << 16);
  __syncthreads();
  for (int i = t; i < L; i += kLabNT) {
    float s = -INFINITY;
    if (i < m) {
      const uint32_t* kr = reinterpret_cast<const uint32_t*>(k + (int64_t)i * kD);
      float a = 0.f;
#pragma unroll 8
      for (int c2 = 0; c2 < kD / 2; ++c2) {
        const uint32_t two = kr[c2];
        a = fmaf(qs[2 * c2], bf16_lo(two), a);
        a = fmaf(qs[2 * c2 + 1], bf16_hi(two), a);
      }
      s = a;
    }
    key[i] = s;
    ids[i] = i;
  }
  __syncthreads();
  // bitonic sort: first = higher score, then lower index
  for (int sz = 2; sz <= L; sz <<= 1) {
    for (int st = sz >> 1; st > 0; st >>= 1) {
      for (int e = t; e < L / 2; e += kLabNT) {
        const int lo = 2 * e - (e & (st - 1));
        const int hi = lo + st;
        const bool up = (lo & sz) == 0;  // this half sorts "first" to the front
        const float ka = key[lo], kb = key[hi];
        const int ia = ids[lo], ib = ids[hi];
        const bool b_first = (kb > ka) || (kb == ka && ib < ia);
        if (b_first == up) {
          key[lo] = kb; key[hi] = ka;
          ids[lo] = ib; ids[hi] = ia;
        }
      }
      __syncthreads();
    }
  }
  const int P = max(1, (m * pos_permille + 999) / 1000);
  float* row = S + (int64_t)j * n;
  for (int r = t; r < m; r += kLabNT) {
    const float v = (r < P) ? ((P == 1) ? s_max : s_max - (s_max - s_min) * (float)r / (float)(P - 1)) : -1.f;
    row[ids[r]] = v;
  }
  for (int i = m + t; i < n; i += kLabNT) row[i] = 0.f;
}

// ------------------------------------------------------------ tiled GEMM
// C[M][N] = alpha * sum_k A(m, k) B(k, n) (+ C if accumulate), fp32.  A and
// B are read through accessor structs; 64 x 64 tiles, 16-deep k steps staged
// in LDS, 256 threads with 4 x 4 outputs each.
struct AccF32 {  // row-major [rows][ld]
  const float* p; int ld;
  __device__ float operator()(int r, int c) const { return p[(int64_t)r * ld + c]; }
};
struct AccF32T {  // element (r, c) of the transpose of a row-major [.][ld]
  const float* p; int ld;
  __device__ float operator()(int r, int c) const { return p[(int64_t)c * ld + r]; }
};
struct AccBf16 {
  const uint16_t* p; int ld;
  __device__ float operator()(int r, int c) const { return __uint_as_float((uint32_t)p[(int64_t)r * ld + c] << 16); }
};
struct AccBf16T {
  const uint16_t* p; int ld;
  __device__ float operator()(int r, int c) const { return __uint_as_float((uint32_t)p[(int64_t)c * ld + r] << 16); }
};
struct AccMask {  // M_ji = [i <= p_j] (rows j, columns i)
  const int32_t* pos; int n;
  __device__ float operator()(int r, int c) const { return c <= min(max(pos[r], 0), n - 1) ? 1.f : 0.f; }
};
struct AccMaskT {  // M^T
  const int32_t* pos; int n;
  __device__ float operator()(int r, int c) const { return r <= min(max(pos[c], 0), n - 1) ? 1.f : 0.f; }
};
struct AccGramMinusI {  // (W^T W - I)[r][c] from a precomputed W^T W
  const float* p; int ld;
  __device__ float operator()(int r, int c) const { return p[(int64_t)r * ld + c] - (r == c ? 1.f : 0.f); }
};

constexpr int kT = 64, kKS = 16;

template <class A, class B>
__global__ __launch_bounds__(256) void gemm_kernel(int M, int N, int K, A a, B b, float* __restrict__ C,
                                                   int ldc, float alpha, int accumulate) {
  __shared__ float as[kKS][kT + 1];
  __shared__ float bs[kKS][kT + 1];
  const int t = threadIdx.x, tx = t & 15, ty = t >> 4;
  const int m0 = blockIdx.y * kT, n0 = blockIdx.x * kT;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += kKS) {
    for (int e = t; e < kT * kKS; e += 256) {
      const int mm = e / kKS, kk = e % kKS;
      as[kk][mm] = (m0 + mm < M && k0 + kk < K) ? a(m0 + mm, k0 + kk) : 0.f;
      const int kb = e / kT, nn = e % kT;
      bs[kb][nn] = (k0 + kb < K && n0 + nn < N) ? b(k0 + kb, n0 + nn) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kKS; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = as[kk][ty * 4 + i];
#pragma unroll
      for (int i = 0; i < 4; ++i) bv[i] = bs[kk][tx * 4 + i];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) acc[i][jj] = fmaf(av[i], bv[jj], acc[i][jj]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int mm = m0 + ty * 4 + i, nn = n0 + tx * 4 + jj;
      if (mm < M && nn < N) {
        float* c = C + (int64_t)mm * ldc + nn;
        *c = alpha * acc[i][jj] + (accumulate ? *c : 0.f);
      }
    }
}

template <class A, class B>
hipError_t gemm(int M, int N, int K, A a, B b, float* C, int ldc, float alpha, bool accumulate, hipStream_t s) {
  dim3 grid((unsigned)((N + kT - 1) / kT), (unsigned)((M + kT - 1) / kT));
  hipLaunchKernelGGL((gemm_kernel<A, B>), grid, dim3(256), 0, s, M, N, K, a, b, C, ldc, alpha, accumulate ? 1 : 0);
  return hipGetLastError();
}

// ------------------------------------------------------------ elementwise
__global__ void tanh_half_kernel(float* z, int64_t count, float half_sigma) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) z[i] = tanhf(half_sigma * z[i]);
}

// rows of X [rows][cols]: out[r] = sum_c X[r][c] (sums S_j) or columns
__global__ void row_sums_kernel(const float* __restrict__ X, int rows, int cols, float* __restrict__ out) {
  const int r = blockIdx.x;
  float a = 0.f;
  for (int c = threadIdx.x; c < cols; c += 256) a += X[(int64_t)r * cols + c];
  __shared__ float red[256];
  red[threadIdx.x] = a;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[r] = red[0];
}
__global__ void col_sums_kernel(const float* __restrict__ X, int rows, int cols, float* __restrict__ out) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= cols) return;
  float a = 0.f;
  for (int r = 0; r < rows; ++r) a += X[(int64_t)r * cols + c];
  out[c] = a;
}

// dZ = (2 eps (rs * H - P) + 2 eta Qb) * (1 - H^2) / 2 per element, where P
// is the pair product (S Hk or S^T Hq) and Qb the balance product (M^T C,
// or null for the queries).  Also the per-row partial loss sums:
// part[row] = rs * ||H_row||^2 (for the similarity term) and
// part2[row] = H_row . P_row.
__global__ void dz_kernel(const float* __restrict__ H, const float* __restrict__ P,
                          const float* __restrict__ Qb, const float* __restrict__ rs, int rows, int r,
                          float eps, float eta, float* __restrict__ dZ, float* __restrict__ part) {
  const int row = blockIdx.x;
  float a1 = 0.f, a2 = 0.f;
  const float w = rs[row];
  for (int c = threadIdx.x; c < r; c += blockDim.x) {
    const int64_t e = (int64_t)row * r + c;
    const float h = H[e], pp = P[e];
    float g = 2.f * eps * (w * h - pp);
    if (Qb) g += 2.f * eta * Qb[e];
    dZ[e] = g * (1.f - h * h) * 0.5f;
    a1 += w * h * h;
    a2 += h * pp;
  }
  __shared__ float red[2][256];
  red[0][threadIdx.x] = a1;
  red[1][threadIdx.x] = a2;
  __syncthreads();
  for (int o = blockDim.x / 2; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) {
      red[0][threadIdx.x] += red[0][threadIdx.x + o];
      red[1][threadIdx.x] += red[1][threadIdx.x + o];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    part[2 * row] = red[0][0];
    part[2 * row + 1] = red[1][0];
  }
}

// Final loss terms and the decorrelation factor, one workgroup (fixed
// order): loss[0..3] = total, similarity, balance, decorrelation;
// fac[0] = 2 lam / ||A||_F (0 when A == 0), A = W^T W - I.
__global__ void loss_kernel(const float* __restrict__ part_q, int J, const float* __restrict__ part_k, int n,
                            const float* __restrict__ Cm, int r, const float* __restrict__ gram,
                            float eps, float eta, float lam, float* __restrict__ loss, float* __restrict__ fac) {
  __shared__ float red[4][256];
  const int t = threadIdx.x;
  float sq = 0.f, sk = 0.f, bal = 0.f, dec = 0.f;
  for (int j = t; j < J; j += 256) sq += part_q[2 * j] - 2.f * part_q[2 * j + 1];
  for (int i = t; i < n; i += 256) sk += part_k[2 * i];
  for (int64_t e = t; e < (int64_t)J * r; e += 256) bal += Cm[e] * Cm[e];
  for (int e = t; e < r * r; e += 256) {
    const float v = gram[e] - ((e / r) == (e % r) ? 1.f : 0.f);
    dec += v * v;
  }
  red[0][t] = sq; red[1][t] = sk; red[2][t] = bal; red[3][t] = dec;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
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

// W -= lr * dW, with dW += fac * W A already accumulated; optional gradient copy
__global__ void update_kernel(float* __restrict__ W, const float* __restrict__ dW, float* __restrict__ grad,
                              int count, float lr) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= count) return;
  const float g = dW[i];
  if (grad) grad[i] = g;
  W[i] -= lr * g;
}

__global__ void scale_add_wa_kernel(float* __restrict__ dW, const float* __restrict__ WA,
                                    const float* __restrict__ fac, int count) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) dW[i] += fac[0] * WA[i];
}

}  // namespace

size_t label_lds_bytes() { return (size_t)(kD + 2 * kMaxLabelKeys) * 4; }

hipError_t launch_hash_labels(const uint16_t* q, const uint16_t* k, const int32_t* q_pos, int J, int n,
                              int pos_permille, float s_max, float s_min, float* S, hipStream_t s) {
  static bool configured = false;
  const size_t lds = label_lds_bytes();
  if (!configured) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&labels_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
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
  p.partq = take((size_t)2 * J);
  p.partk = take((size_t)2 * n);
  p.fac = take(4);
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
  float *WA = F(p.wa), *partq = F(p.partq), *partk = F(p.partk), *fac = F(p.fac);
  hipError_t e;
#define HATA_TRY(x) do { e = (x); if (e != hipSuccess) return e; } while (0)
  // H = tanh(sigma/2 * X W)
  HATA_TRY(gemm(J, r, kD, AccBf16{q, kD}, AccF32{W, r}, Hq, r, 1.f, false, s));
  HATA_TRY(gemm(n, r, kD, AccBf16{k, kD}, AccF32{W, r}, Hk, r, 1.f, false, s));
  {
    const int64_t a = (int64_t)J * r, b = (int64_t)n * r;
    hipLaunchKernelGGL(tanh_half_kernel, dim3((unsigned)((a + 255) / 256)), dim3(256), 0, s, Hq, a, 0.5f * sigma);
    hipLaunchKernelGGL(tanh_half_kernel, dim3((unsigned)((b + 255) / 256)), dim3(256), 0, s, Hk, b, 0.5f * sigma);
    HATA_TRY(hipGetLastError());
  }
  // pair products, label sums, balance products
  HATA_TRY(gemm(J, r, n, AccF32{S, n}, AccF32{Hk, r}, SHk, r, 1.f, false, s));
  HATA_TRY(gemm(n, r, J, AccF32T{S, n}, AccF32{Hq, r}, StHq, r, 1.f, false, s));
  HATA_TRY(gemm(J, r, n, AccMask{q_pos, n}, AccF32{Hk, r}, Cm, r, 1.f, false, s));
  HATA_TRY(gemm(n, r, J, AccMaskT{q_pos, n}, AccF32{Cm, r}, MtC, r, 1.f, false, s));
  hipLaunchKernelGGL(row_sums_kernel, dim3(J), dim3(256), 0, s, S, J, n, rs);
  hipLaunchKernelGGL(col_sums_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, S, J, n, cs);
  HATA_TRY(hipGetLastError());
  // dZ and the per-row loss parts
  hipLaunchKernelGGL(dz_kernel, dim3(J), dim3(128), 0, s, Hq, SHk, (const float*)nullptr, rs, J, r, eps, eta, dZq, partq);
  hipLaunchKernelGGL(dz_kernel, dim3(n), dim3(128), 0, s, Hk, StHq, MtC, cs, n, r, eps, eta, dZk, partk);
  HATA_TRY(hipGetLastError());
  // dW = sigma (Q^T dZq + K^T dZk)
  HATA_TRY(gemm(kD, r, J, AccBf16T{q, kD}, AccF32{dZq, r}, dW, r, sigma, false, s));
  HATA_TRY(gemm(kD, r, n, AccBf16T{k, kD}, AccF32{dZk, r}, dW, r, sigma, true, s));
  // decorrelation: gram = W^T W, WA = W (gram - I), dW += 2 lam / ||A|| * WA
  HATA_TRY(gemm(r, r, kD, AccF32T{W, r}, AccF32{W, r}, gram, r, 1.f, false, s));
  HATA_TRY(gemm(kD, r, r, AccF32{W, r}, AccGramMinusI{gram, r}, WA, r, 1.f, false, s));
  hipLaunchKernelGGL(loss_kernel, dim3(1), dim3(256), 0, s, partq, J, partk, n, Cm, r, gram, eps, eta, lam, loss, fac);
  hipLaunchKernelGGL(scale_add_wa_kernel, dim3((kD * r + 255) / 256), dim3(256), 0, s, dW, WA, fac, kD * r);
  hipLaunchKernelGGL(update_kernel, dim3((kD * r + 255) / 256), dim3(256), 0, s, W, dW, grad, kD * r, lr);
  return hipGetLastError();
#undef HATA_TRY
}

}  // namespace hata
