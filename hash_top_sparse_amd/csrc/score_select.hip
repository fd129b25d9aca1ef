// score_select.hip -- Hamming scores with GQA sum, and top-k selection.
//
// HATA paper notes, section "Key design: Decode-stage algorithm": the score of
// a cached key is bitcount(xor(query code, key code)); under GQA the scores
// of the query heads that share one KV cache are aggregated (summed here);
// the top-k tokens -- smallest summed distance, ties to the lower index -- are
// selected.  Section "Hardware-efficient optimisation": XOR + popcount with
// coalesced memory access.
#include "hata_device.hpp"
#include "hata_launch.hpp"

namespace hata {

namespace {

constexpr int kHamTPT = 8;  // tokens per thread in the staged Hamming kernel

// PAGED: kc is a page pool addressed through pm.
template <int G, int R, bool PAGED>
__global__ __launch_bounds__(kNT) void hamming_kernel(const uint64_t* __restrict__ qc,
                                                      const uint64_t* __restrict__ kc, int Hq,
                                                      int Hkv, int64_t cap,
                                                      const int32_t* __restrict__ seq_lens,
                                                      uint16_t* __restrict__ scores,
                                                      int64_t sstride, PageMap pm) {
  const int t = threadIdx.x;
  const int unit = blockIdx.y;
  const int b = unit / Hkv, h = unit - b * Hkv;
  int64_t n = seq_lens[b];
  if (n < 0) n = 0;
  if (n > cap) n = cap;
  if (n > sstride) n = sstride;
  const int64_t i0 = (int64_t)blockIdx.x * (kNT * kHamTPT);
  if (i0 >= n) return;

  constexpr int W64 = Width<R>::W64, W32 = Width<R>::W32;
  uint32_t qw[G][W32];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const uint64_t* qp = qc + ((int64_t)b * Hq + (int64_t)h * G + g) * W64;
#pragma unroll
    for (int w = 0; w < W32; ++w) qw[g][w] = (uint32_t)(qp[w >> 1] >> ((w & 1) * 32));
  }
  QMasks<G, R> m;
  build_qmasks<G, R>(qw, m);

  const uint64_t* src = kc + ((int64_t)b * Hkv + h) * cap * W64;
  uint16_t* dst = scores + ((int64_t)b * Hkv + h) * sstride;
  CodeRow<R> c[kHamTPT];
#pragma unroll
  for (int j = 0; j < kHamTPT; ++j) {
    const int64_t i = i0 + j * kNT + t;
    if (i < n) c[j] = PAGED ? load_code<R>(kc, pm.row(b, h, Hkv, i)) : load_code<R>(src, i);
  }
#pragma unroll
  for (int j = 0; j < kHamTPT; ++j) {
    const int64_t i = i0 + j * kNT + t;
    if (i < n) {
      uint32_t cw[W32];
      code_words<R>(c[j], cw);
      dst[i] = (uint16_t)gqa_hamming_w<G, R>(cw, m);
    }
  }
}

// One 1024-thread workgroup per unit: histogram of the scores, threshold T =
// smallest s with count(score <= s) >= k, then an ordered compaction that
// keeps every score < T and the lowest-index (k - count(< T)) ties at T.
constexpr int kTopkNT = 1024;
constexpr int kMaxBins = 8 * 256 + 1;  // G * r + 1 at G = 8, r = 256

__device__ __forceinline__ uint32_t block_excl_scan_1024(uint32_t v, uint32_t* tmp, uint32_t* total) {
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  (void)lane;
  const uint32_t inc = wave_incl_scan_u32(v);
  if (lane == 63) tmp[wv] = inc;
  __syncthreads();
  uint32_t base = 0, all = 0;
#pragma unroll
  for (int i = 0; i < kTopkNT / 64; ++i) {
    const uint32_t s = tmp[i];
    base += (i < wv) ? s : 0u;
    all += s;
  }
  __syncthreads();
  *total = all;
  return base + inc - v;
}

__global__ __launch_bounds__(kTopkNT) void topk_kernel(const uint16_t* __restrict__ scores,
                                                       int64_t sstride, int Hkv, int64_t cap,
                                                       const int32_t* __restrict__ seq_lens, int k,
                                                       int max_score, int32_t* __restrict__ idx) {
  __shared__ uint32_t hist[kMaxBins + 3];
  __shared__ uint32_t tmp[kTopkNT / 64];
  __shared__ uint32_t stat[2];
  const int t = threadIdx.x;
  const int unit = blockIdx.x;
  const int b = unit / Hkv;
  int64_t n64 = seq_lens[b];
  if (n64 < 0) n64 = 0;
  if (n64 > cap) n64 = cap;
  if (n64 > sstride) n64 = sstride;
  const int n = (int)n64;
  const int nb = max_score + 1;
  const uint16_t* sc = scores + (int64_t)unit * sstride;
  int32_t* out = idx + (int64_t)unit * k;

  for (int i = t; i < nb; i += kTopkNT) hist[i] = 0;
  if (t < 2) stat[t] = 0;
  __syncthreads();
  for (int i = t; i < n; i += kTopkNT) {
    const int s = min((int)sc[i], max_score);
    atomicAdd(&hist[s], 1u);
  }
  __syncthreads();
  // cumulative histogram: thread t owns bins [t*bpt, (t+1)*bpt)
  const int bpt = (nb + kTopkNT - 1) / kTopkNT;
  uint32_t loc = 0;
  for (int j = 0; j < bpt; ++j) {
    const int s = t * bpt + j;
    if (s < nb) loc += hist[s];
  }
  uint32_t tot;
  uint32_t run = block_excl_scan_1024(loc, tmp, &tot);
  uint32_t below_k = 0;  // bins s with cum(s) < k
  for (int j = 0; j < bpt; ++j) {
    const int s = t * bpt + j;
    if (s < nb) {
      run += hist[s];
      hist[s] = run;
      below_k += (run < (uint32_t)k) ? 1u : 0u;
    }
  }
  atomicAdd(&stat[0], below_k);
  __syncthreads();
  int T = (int)stat[0];
  if (T >= nb) T = nb - 1;  // fewer than k tokens: keep everything
  const uint32_t lt_total = T > 0 ? hist[T - 1] : 0u;
  const uint32_t quota = (uint32_t)k - lt_total;  // ties to keep (may exceed the tie count)

  // ordered compaction over contiguous per-thread ranges
  const int per = (n + kTopkNT - 1) / kTopkNT;
  const int i_begin = min(n, t * per), i_end = min(n, i_begin + per);
  uint32_t lt = 0, eq = 0;
  for (int i = i_begin; i < i_end; ++i) {
    const int s = min((int)sc[i], max_score);
    lt += (s < T);
    eq += (s == T);
  }
  uint32_t dummy;
  uint32_t lt_before = block_excl_scan_1024(lt, tmp, &dummy);
  uint32_t eq_before = block_excl_scan_1024(eq, tmp, &dummy);
  for (int i = i_begin; i < i_end; ++i) {
    const int s = min((int)sc[i], max_score);
    if (s < T) {
      out[lt_before + min(eq_before, quota)] = i;
      ++lt_before;
    } else if (s == T) {
      if (eq_before < quota) out[lt_before + eq_before] = i;
      ++eq_before;
    }
  }
  const int m = min(k, n);
  for (int j = m + t; j < k; j += kTopkNT) out[j] = -1;
}

}  // namespace

template <int G, int R>
static void launch_hamming_gr(const uint64_t* qc, const uint64_t* kc, int Hq, int Hkv, int64_t cap,
                              const int32_t* seq_lens, uint16_t* scores, int64_t sstride, dim3 grid,
                              const PageMap* pm, hipStream_t s) {
  if (pm && pm->bt)
    hipLaunchKernelGGL((hamming_kernel<G, R, true>), grid, dim3(kNT), 0, s, qc, kc, Hq, Hkv, cap, seq_lens,
                       scores, sstride, *pm);
  else
    hipLaunchKernelGGL((hamming_kernel<G, R, false>), grid, dim3(kNT), 0, s, qc, kc, Hq, Hkv, cap, seq_lens,
                       scores, sstride, PageMap());
}

template <int R>
static hipError_t launch_hamming_r(const uint64_t* qc, const uint64_t* kc, int G, int Hq, int Hkv,
                                   int64_t cap, const int32_t* seq_lens, uint16_t* scores, int64_t sstride,
                                   dim3 grid, const PageMap* pm, hipStream_t s) {
  switch (G) {
    case 1: launch_hamming_gr<1, R>(qc, kc, Hq, Hkv, cap, seq_lens, scores, sstride, grid, pm, s); break;
    case 2: launch_hamming_gr<2, R>(qc, kc, Hq, Hkv, cap, seq_lens, scores, sstride, grid, pm, s); break;
    case 4: launch_hamming_gr<4, R>(qc, kc, Hq, Hkv, cap, seq_lens, scores, sstride, grid, pm, s); break;
    case 8: launch_hamming_gr<8, R>(qc, kc, Hq, Hkv, cap, seq_lens, scores, sstride, grid, pm, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_hamming(const uint64_t* qc, const uint64_t* kc, int B, int Hq, int Hkv,
                          int64_t cap, const int32_t* seq_lens, int64_t max_len, uint16_t* scores,
                          int64_t sstride, hipStream_t s, int r, const PageMap* pm) {
  const int G = Hq / Hkv;
  const int64_t per_block = (int64_t)kNT * kHamTPT;
  dim3 grid((unsigned)((max_len + per_block - 1) / per_block), (unsigned)(B * Hkv));
  switch (r) {
    case 32: return launch_hamming_r<32>(qc, kc, G, Hq, Hkv, cap, seq_lens, scores, sstride, grid, pm, s);
    case 64: return launch_hamming_r<64>(qc, kc, G, Hq, Hkv, cap, seq_lens, scores, sstride, grid, pm, s);
    case 256: return launch_hamming_r<256>(qc, kc, G, Hq, Hkv, cap, seq_lens, scores, sstride, grid, pm, s);
    default: return launch_hamming_r<128>(qc, kc, G, Hq, Hkv, cap, seq_lens, scores, sstride, grid, pm, s);
  }
}

hipError_t launch_topk(const uint16_t* scores, int64_t sstride, int B, int Hkv, int64_t cap,
                       const int32_t* seq_lens, int k, int max_score, int32_t* idx, hipStream_t s) {
  if (max_score + 1 > kMaxBins) return hipErrorInvalidValue;
  hipLaunchKernelGGL(topk_kernel, dim3(B * Hkv), dim3(kTopkNT), 0, s, scores, sstride, Hkv, cap,
                     seq_lens, k, max_score, idx);
  return hipGetLastError();
}

}  // namespace hata
