// attention.hip -- gather-fused split-K flash-decode (sparse and dense).
//
// HATA paper notes, section "Overall framework" (decode phase: exact attention
// over the selected KV pairs only) and section "Hardware-efficient
// optimisation" (the gather of the selected rows is fused into the
// FlashAttention kernel instead of materialising a gathered copy).
//
// Each workgroup takes a slice of one unit's row list, reads each K/V row
// once for all G query heads of the unit (16 lanes per row, 8 channels per
// lane, 16-byte loads), keeps an online softmax per head and writes one
// (max, sum, acc[128]) record per head; a second kernel merges the records
// of a unit by log-sum-exp in a fixed order.  The dense baseline is the same
// kernel with the row list 0..n-1.
#include "hata_device.hpp"
#include "hata_launch.hpp"

namespace hata {

namespace {

constexpr int kUnroll = 4;  // rows in flight per 16-lane group

int splits_for(int units, int64_t rows, bool dense, int* rows_per_split) {
  int64_t rps;
  if (!dense) {
    rps = 32;
  } else {
    // about 4 workgroups per CU over the whole launch, at least 256 rows each
    int64_t target = (4 * 256 + units - 1) / units;
    if (target < 1) target = 1;
    rps = (rows + target - 1) / target;
    if (rps < 256) rps = 256;
    rps = (rps + 63) / 64 * 64;
  }
  int64_t sp = (rows + rps - 1) / rps;
  if (sp < 1) sp = 1;
  *rows_per_split = (int)rps;
  return (int)sp;
}

// PAGED: K and V are page pools addressed through pm.
template <int G, bool PAGED>
__global__ __launch_bounds__(kNT) void attn_partial_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    int Hq, int Hkv, int64_t cap, const int32_t* __restrict__ idx, int k,
    const int32_t* __restrict__ seq_lens, int rows_per_split, int splits, float scale,
    float* __restrict__ part, PageMap pm) {
  __shared__ float red[kMergeFloats<G>];
  const int t = threadIdx.x, slot = t >> 4, sub = t & 15;
  const int unit = blockIdx.y, split = blockIdx.x;
  const int b = unit / Hkv, h = unit - b * Hkv;
  int64_t n = cap;
  if (!idx) {
    n = seq_lens[b];
    if (n < 0) n = 0;
    if (n > cap) n = cap;
  }
  const int64_t total = idx ? (int64_t)k : n;
  const int64_t r_begin = (int64_t)split * rows_per_split;
  const int64_t r_end = r_begin + rows_per_split < total ? r_begin + rows_per_split : total;

  float qreg[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const uint4 v = *reinterpret_cast<const uint4*>(q + ((int64_t)b * Hq + (int64_t)h * G + g) * kD + sub * 8);
    unpack8(v, qreg[g]);
  }
  const int64_t row0 = PAGED ? 0 : ((int64_t)b * Hkv + h) * cap;
  const uint16_t* Kb = K + row0 * kD + sub * 8;
  const uint16_t* Vb = V + row0 * kD + sub * 8;
  const int32_t* ib = idx ? idx + (int64_t)unit * k : nullptr;

  SoftmaxState<G> st;
  st.init();
  for (int64_t r0 = r_begin + slot; r0 < r_end; r0 += 16 * kUnroll) {
    uint4 kv[kUnroll], vv[kUnroll];
    bool valid[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t r = r0 + 16 * u;
      kv[u] = make_uint4(0, 0, 0, 0);
      vv[u] = make_uint4(0, 0, 0, 0);
      valid[u] = false;
      if (r < r_end) {
        const int64_t tok = ib ? (int64_t)ib[r] : r;
        if (tok >= 0 && tok < n) {
          valid[u] = true;
          const int64_t pr = PAGED ? pm.row(b, h, Hkv, tok) : tok;
          kv[u] = *reinterpret_cast<const uint4*>(Kb + pr * kD);
          vv[u] = *reinterpret_cast<const uint4*>(Vb + pr * kD);
        }
      }
    }
    attend_block<G, kUnroll>(st, qreg, kv, vv, valid, scale);
  }
  merge_wg<G>(st, red);
  float* dst = part + ((int64_t)unit * splits + split) * (G * kRec);
  for (int e = t; e < G * kRec; e += kNT) dst[e] = red[e];
}

// Log-sum-exp merge of a unit's split records.  One workgroup per (unit,
// head, 16-channel slice); lane (s16, ch) = (t / 16, t % 16) walks splits
// s16, s16+16, ... so each thread issues only a few independent loads, and
// the 16 split lanes are merged through LDS in fixed order.
template <int G>
__global__ __launch_bounds__(kNT) void attn_combine_kernel(const float* __restrict__ part,
                                                           int splits, int Hq, int Hkv,
                                                           float* __restrict__ out) {
  __shared__ float sm[16][16];
  __shared__ float sl[16][16];
  __shared__ float sa[16][16];
  const int t = threadIdx.x, s16 = t >> 4, ch = t & 15;
  const int unit = blockIdx.x, g = blockIdx.y, c = blockIdx.z * 16 + ch;
  const int b = unit / Hkv, h = unit - b * Hkv;
  const float* src = part + (int64_t)unit * splits * (G * kRec) + g * kRec;
  float M = -INFINITY;
  for (int s = s16; s < splits; s += 16) M = fmaxf(M, src[(int64_t)s * G * kRec]);
  float L = 0.f, A = 0.f;
  if (M != -INFINITY) {
    for (int s = s16; s < splits; s += 16) {
      const float* r = src + (int64_t)s * G * kRec;
      const float f = __expf(r[0] - M);
      L = fmaf(r[1], f, L);
      A = fmaf(r[2 + c], f, A);
    }
  }
  sm[s16][ch] = M;
  sl[s16][ch] = L;
  sa[s16][ch] = A;
  __syncthreads();
  if (s16 == 0) {
    float Mg = -INFINITY;
    for (int i = 0; i < 16; ++i) Mg = fmaxf(Mg, sm[i][ch]);
    float Lg = 0.f, Ag = 0.f;
    if (Mg != -INFINITY) {
      for (int i = 0; i < 16; ++i) {
        const float f = (sm[i][ch] == -INFINITY) ? 0.f : __expf(sm[i][ch] - Mg);
        Lg = fmaf(sl[i][ch], f, Lg);
        Ag = fmaf(sa[i][ch], f, Ag);
      }
    }
    out[((int64_t)b * Hq + (int64_t)h * G + g) * kD + c] = (Lg > 0.f) ? Ag / Lg : 0.f;
  }
}

template <int G>
hipError_t launch_attention_g(const uint16_t* q, const uint16_t* K, const uint16_t* V, int B,
                              int Hq, int Hkv, int64_t cap, const int32_t* idx, int k,
                              const int32_t* seq_lens, int64_t max_len, float scale, float* out,
                              float* part, hipStream_t s, const PageMap* pm) {
  const int U = B * Hkv;
  int rps;
  const int splits = splits_for(U, idx ? (int64_t)k : max_len, idx == nullptr, &rps);
  if (pm && pm->bt)
    hipLaunchKernelGGL((attn_partial_kernel<G, true>), dim3(splits, U), dim3(kNT), 0, s, q, K, V, Hq, Hkv,
                       cap, idx, k, seq_lens, rps, splits, scale, part, *pm);
  else
    hipLaunchKernelGGL((attn_partial_kernel<G, false>), dim3(splits, U), dim3(kNT), 0, s, q, K, V, Hq, Hkv,
                       cap, idx, k, seq_lens, rps, splits, scale, part, PageMap());
  hipLaunchKernelGGL(attn_combine_kernel<G>, dim3(U, G, kD / 16), dim3(kNT), 0, s, part, splits, Hq,
                     Hkv, out);
  return hipGetLastError();
}

}  // namespace

size_t attn_part_floats(int B, int Hkv, int G, int64_t max_rows_sparse_or_dense) {
  // sized for the larger of the sparse and dense split plans
  int rps;
  const int U = B * Hkv;
  const int sp_dense = splits_for(U, max_rows_sparse_or_dense, true, &rps);
  const int sp_sparse = splits_for(U, max_rows_sparse_or_dense, false, &rps);
  const int sp = sp_dense > sp_sparse ? sp_dense : sp_sparse;
  return (size_t)U * sp * G * kRec;
}

hipError_t launch_attention(const uint16_t* q, const uint16_t* K, const uint16_t* V, int B, int Hq,
                            int Hkv, int64_t cap, const int32_t* idx, int k,
                            const int32_t* seq_lens, int64_t max_len, float scale, float* out,
                            float* part, hipStream_t s, const PageMap* pm) {
  switch (Hq / Hkv) {
    case 1: return launch_attention_g<1>(q, K, V, B, Hq, Hkv, cap, idx, k, seq_lens, max_len, scale, out, part, s, pm);
    case 2: return launch_attention_g<2>(q, K, V, B, Hq, Hkv, cap, idx, k, seq_lens, max_len, scale, out, part, s, pm);
    case 4: return launch_attention_g<4>(q, K, V, B, Hq, Hkv, cap, idx, k, seq_lens, max_len, scale, out, part, s, pm);
    case 8: return launch_attention_g<8>(q, K, V, B, Hq, Hkv, cap, idx, k, seq_lens, max_len, scale, out, part, s, pm);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace hata
