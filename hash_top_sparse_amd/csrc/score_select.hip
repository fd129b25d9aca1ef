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

// PAGED: kc is a page pool addressed through pm.  HIST: also add this
// workgroup's score histogram (bins 0..G r) into hist[unit][G r + 1] (for the
// many-workgroup top-k; hist zeroed beforehand).
template <int G, int R, bool PAGED, bool HIST>
__global__ __launch_bounds__(kNT) void hamming_kernel(const uint32_t* __restrict__ qc,
                                                      const uint32_t* __restrict__ kc, int Hq,
                                                      int Hkv, int64_t cap,
                                                      const int32_t* __restrict__ seq_lens,
                                                      uint16_t* __restrict__ scores,
                                                      int64_t sstride, PageMap pm,
                                                      uint32_t* __restrict__ hist) {
  const int t = threadIdx.x;
  const int unit = blockIdx.y;
  const int b = unit / Hkv, h = unit - b * Hkv;
  int64_t n = seq_lens[b];
  if (n < 0) n = 0;
  if (n > cap) n = cap;
  if (n > sstride) n = sstride;
  const int64_t i0 = (int64_t)blockIdx.x * (kNT * kHamTPT);
  if (i0 >= n) return;

  constexpr int W32 = Width<R>::W32;
  uint32_t qw[G][W32];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const uint32_t* qp = qc + ((int64_t)b * Hq + (int64_t)h * G + g) * W32;
#pragma unroll
    for (int w = 0; w < W32; ++w) qw[g][w] = qp[w];
  }
  QMasks<G, R> m;
  build_qmasks<G, R>(qw, m);

  const uint32_t* src = kc + ((int64_t)b * Hkv + h) * cap * W32;
  uint16_t* dst = scores + ((int64_t)b * Hkv + h) * sstride;
  CodeRow<R> c[kHamTPT];
#pragma unroll
  for (int j = 0; j < kHamTPT; ++j) {
    const int64_t i = i0 + j * kNT + t;
    if (i < n) c[j] = PAGED ? load_code<R>(kc, pm.row(b, h, Hkv, i)) : load_code<R>(src, i);
  }
  constexpr int NB = G * R + 1;
  __shared__ uint32_t bins[HIST ? NB : 1];
  if constexpr (HIST) {
    for (int e = t; e < NB; e += kNT) bins[e] = 0;
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < kHamTPT; ++j) {
    const int64_t i = i0 + j * kNT + t;
    if (i < n) {
      uint32_t cw[W32];
      code_words<R>(c[j], cw);
      const uint32_t sv = gqa_hamming_w<G, R>(cw, m);
      dst[i] = (uint16_t)sv;
      if constexpr (HIST) atomicAdd(&bins[sv], 1u);
    }
  }
  if constexpr (HIST) {
    __syncthreads();
    for (int e = t; e < NB; e += kNT)
      if (bins[e]) atomicAdd(&hist[(int64_t)unit * NB + e], bins[e]);
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

// ---- multi-workgroup top-k for long sequences: the same selection as
// topk_kernel in four passes over chunks of kTkChunk scores.
//   1. unit histogram (per-chunk LDS histograms added into the unit's)
//   2. threshold T and tie quota per unit; -1 padding past min(k, n)
//   3. per chunk: counts of scores < T and == T
//   4. per chunk: ordered compaction at offset (kept rows in earlier chunks),
//      a row's slot being (#rows < T before it) + min(#ties before it, quota)
constexpr int kTkChunk = 4096;

__device__ __forceinline__ int unit_len(const int32_t* seq_lens, int b, int64_t cap, int64_t sstride) {
  int64_t n = seq_lens[b];
  if (n < 0) n = 0;
  if (n > cap) n = cap;
  if (n > sstride) n = sstride;
  return (int)n;
}

__global__ __launch_bounds__(kNT) void topk_hist_kernel(const uint16_t* __restrict__ scores, int64_t sstride,
                                                        int Hkv, int64_t cap, const int32_t* __restrict__ seq_lens,
                                                        int max_score, uint32_t* __restrict__ hist) {
  __shared__ uint32_t h[kMaxBins];
  const int t = threadIdx.x, unit = blockIdx.y;
  const int n = unit_len(seq_lens, unit / Hkv, cap, sstride);
  const int i0 = blockIdx.x * kTkChunk;
  if (i0 >= n) return;
  const int nb = max_score + 1;
  for (int i = t; i < nb; i += kNT) h[i] = 0;
  __syncthreads();
  const uint16_t* sc = scores + (int64_t)unit * sstride;
  const int i1 = min(n, i0 + kTkChunk);
  for (int i = i0 + t; i < i1; i += kNT) atomicAdd(&h[min((int)sc[i], max_score)], 1u);
  __syncthreads();
  for (int i = t; i < nb; i += kNT)
    if (h[i]) atomicAdd(&hist[(int64_t)unit * nb + i], h[i]);
}

// T = smallest score s with count(<= s) >= k (the top bin when the unit has
// fewer than k scores) and the tie quota k - count(< T), from the unit's
// histogram; every thread of the workgroup gets them.
__device__ __forceinline__ void unit_threshold(const uint32_t* __restrict__ hu, int nb, int k, uint32_t* tmp,
                                               uint32_t* stat, int* T_out, uint32_t* quota_out) {
  const int t = threadIdx.x;
  const int bpt = (nb + kNT - 1) / kNT;
  uint32_t loc = 0;
  for (int j = 0; j < bpt; ++j) {
    const int s = t * bpt + j;
    if (s < nb) loc += hu[s];
  }
  if (t == 0) *stat = 0;
  uint32_t tot;
  uint32_t run = block_excl_scan_u32(loc, tmp, &tot);
  uint32_t below_k = 0;  // bins with cum < k
  for (int j = 0; j < bpt; ++j) {
    const int s = t * bpt + j;
    if (s < nb) {
      run += hu[s];
      below_k += (run < (uint32_t)k) ? 1u : 0u;
    }
  }
  atomicAdd(stat, below_k);
  __syncthreads();
  int T = (int)*stat;
  if (T >= nb) T = nb - 1;  // fewer than k tokens: keep everything
  uint32_t lt = 0;
  for (int j = 0; j < bpt; ++j) {
    const int s = t * bpt + j;
    if (s < T) lt += hu[s];
  }
  uint32_t lt_total;
  (void)block_excl_scan_u32(lt, tmp, &lt_total);
  *T_out = T;
  *quota_out = (uint32_t)k - lt_total;
}

// One workgroup per unit: T and the tie quota into params, -1 padding past
// min(k, n).
__global__ __launch_bounds__(kNT) void topk_thresh_kernel(const uint32_t* __restrict__ hist, int nb, int Hkv,
                                                          int64_t cap, int64_t sstride,
                                                          const int32_t* __restrict__ seq_lens, int k,
                                                          uint32_t* __restrict__ params, int32_t* __restrict__ idx) {
  __shared__ uint32_t tmp[16];
  __shared__ uint32_t stat;
  const int t = threadIdx.x, unit = blockIdx.x;
  const int n = unit_len(seq_lens, unit / Hkv, cap, sstride);
  int T;
  uint32_t quota;
  unit_threshold(hist + (int64_t)unit * nb, nb, k, tmp, &stat, &T, &quota);
  if (t == 0) {
    params[2 * unit] = (uint32_t)T;
    params[2 * unit + 1] = quota;
  }
  int32_t* out = idx + (int64_t)unit * k;
  for (int j = min(k, n) + t; j < k; j += kNT) out[j] = -1;
}

// This thread's 16 consecutive scores from row b0 (rows past n read as
// max_score + 1, which no threshold selects).
__device__ __forceinline__ void load16(const uint16_t* sc, int b0, int n, int max_score, int (&v)[16]) {
  if (b0 + 16 <= n && (reinterpret_cast<uintptr_t>(sc + b0) & 15) == 0) {
    const uint4 x = *reinterpret_cast<const uint4*>(sc + b0);
    const uint4 y = *reinterpret_cast<const uint4*>(sc + b0 + 8);
    const uint32_t w[8] = {x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      v[2 * j] = min((int)(w[j] & 0xFFFFu), max_score);
      v[2 * j + 1] = min((int)(w[j] >> 16), max_score);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = b0 + j < n ? min((int)sc[b0 + j], max_score) : max_score + 1;
  }
}

// Per chunk: counts of scores < T and == T.  own_threshold: T and the tie
// quota come from the unit histogram (unit_threshold, computed while this
// thread's scores load), and chunk 0 stores them in params and writes the -1
// padding past min(k, n); otherwise they are read from params.
__global__ __launch_bounds__(kNT) void topk_count_kernel(const uint16_t* __restrict__ scores, int64_t sstride,
                                                         int Hkv, int64_t cap, const int32_t* __restrict__ seq_lens,
                                                         int max_score, uint32_t* __restrict__ params,
                                                         int chunks, uint32_t* __restrict__ cnt,
                                                         const uint32_t* __restrict__ hist, int k,
                                                         int own_threshold, int32_t* __restrict__ idx) {
  __shared__ uint32_t tmp[16];
  __shared__ uint32_t stat;
  const int t = threadIdx.x, unit = blockIdx.y, c = blockIdx.x;
  const int n = unit_len(seq_lens, unit / Hkv, cap, sstride);
  const int i0 = c * kTkChunk;
  if (own_threshold && c == 0) {
    int32_t* out = idx + (int64_t)unit * k;
    for (int j = min(k, n) + t; j < k; j += kNT) out[j] = -1;
  }
  if (i0 >= n) return;  // chunks past the end are never summed
  int v[16];
  load16(scores + (int64_t)unit * sstride, i0 + 16 * t, n, max_score, v);
  int T;
  if (own_threshold) {
    uint32_t quota;
    unit_threshold(hist + (int64_t)unit * (max_score + 1), max_score + 1, k, tmp, &stat, &T, &quota);
    if (c == 0 && t == 0) {
      params[2 * unit] = (uint32_t)T;
      params[2 * unit + 1] = quota;
    }
  } else {
    T = (int)params[2 * unit];
  }
  uint32_t lt = 0, eq = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    lt += v[j] < T;
    eq += v[j] == T;
  }
  uint32_t both;  // a chunk holds at most 4096 scores: both counts fit in 16 bits
  (void)block_excl_scan_u32(lt | (eq << 16), tmp, &both);
  if (t == 0) {
    cnt[((int64_t)unit * chunks + c) * 2] = both & 0xFFFFu;
    cnt[((int64_t)unit * chunks + c) * 2 + 1] = both >> 16;
  }
}

__global__ __launch_bounds__(kNT) void topk_compact_kernel(const uint16_t* __restrict__ scores, int64_t sstride,
                                                           int Hkv, int64_t cap,
                                                           const int32_t* __restrict__ seq_lens, int max_score,
                                                           const uint32_t* __restrict__ params, int chunks,
                                                           const uint32_t* __restrict__ cnt, int k,
                                                           int32_t* __restrict__ idx) {
  __shared__ uint32_t tmp[16];
  const int t = threadIdx.x, unit = blockIdx.y, c = blockIdx.x;
  const int n = unit_len(seq_lens, unit / Hkv, cap, sstride);
  const int i0 = c * kTkChunk;
  if (i0 >= n) return;
  const int b0 = i0 + 16 * t;
  int v[16];
  load16(scores + (int64_t)unit * sstride, b0, n, max_score, v);
  const int T = (int)params[2 * unit];
  const uint32_t quota = params[2 * unit + 1];
  // rows < T and ties in the chunks before this one
  uint32_t lt_p = 0, eq_p = 0;
  for (int cc = t; cc < c; cc += kNT) {
    lt_p += cnt[((int64_t)unit * chunks + cc) * 2];
    eq_p += cnt[((int64_t)unit * chunks + cc) * 2 + 1];
  }
  uint32_t lt_before, eq_before;
  (void)block_excl_scan_u32(lt_p, tmp, &lt_before);
  (void)block_excl_scan_u32(eq_p, tmp, &eq_before);
  // this chunk: thread t owns rows b0 .. b0 + 15 in order; a row's slot is
  // #(< T) before it + min(#(= T) before it, quota)
  uint32_t lt = 0, eq = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    lt += v[j] < T;
    eq += v[j] == T;
  }
  uint32_t dummy;
  const uint32_t pre = block_excl_scan_u32(lt | (eq << 16), tmp, &dummy);
  uint32_t ltb = lt_before + (pre & 0xFFFFu);
  uint32_t eqb = eq_before + (pre >> 16);
  int32_t* out = idx + (int64_t)unit * k;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (v[j] < T) {
      out[ltb + min(eqb, quota)] = b0 + j;
      ++ltb;
    } else if (v[j] == T) {
      if (eqb < quota) out[ltb + eqb] = b0 + j;
      ++eqb;
    }
  }
}

}  // namespace

size_t topk_scratch_bytes(int B, int Hkv, int64_t max_len, int max_score) {
  const size_t U = (size_t)B * Hkv;
  const size_t chunks = (size_t)((max_len + kTkChunk - 1) / kTkChunk);
  const size_t nb = (size_t)max_score + 1;
  return (U * nb + U * 2 + U * chunks * 2) * 4;
}

template <int G, int R>
static void launch_hamming_gr(const uint32_t* qc, const uint32_t* kc, int Hq, int Hkv, int64_t cap,
                              const int32_t* seq_lens, uint16_t* scores, int64_t sstride, dim3 grid,
                              const PageMap* pm, uint32_t* hist, hipStream_t s) {
  const bool paged = pm && pm->bt;
  const PageMap m = paged ? *pm : PageMap();
  if (paged && hist)
    hipLaunchKernelGGL((hamming_kernel<G, R, true, true>), grid, dim3(kNT), 0, s, qc, kc, Hq, Hkv, cap, seq_lens,
                       scores, sstride, m, hist);
  else if (paged)
    hipLaunchKernelGGL((hamming_kernel<G, R, true, false>), grid, dim3(kNT), 0, s, qc, kc, Hq, Hkv, cap, seq_lens,
                       scores, sstride, m, hist);
  else if (hist)
    hipLaunchKernelGGL((hamming_kernel<G, R, false, true>), grid, dim3(kNT), 0, s, qc, kc, Hq, Hkv, cap, seq_lens,
                       scores, sstride, m, hist);
  else
    hipLaunchKernelGGL((hamming_kernel<G, R, false, false>), grid, dim3(kNT), 0, s, qc, kc, Hq, Hkv, cap, seq_lens,
                       scores, sstride, m, hist);
}

template <int R>
static hipError_t launch_hamming_r(const uint32_t* qc, const uint32_t* kc, int G, int Hq, int Hkv,
                                   int64_t cap, const int32_t* seq_lens, uint16_t* scores, int64_t sstride,
                                   dim3 grid, const PageMap* pm, uint32_t* hist, hipStream_t s) {
  switch (G) {
    case 1: launch_hamming_gr<1, R>(qc, kc, Hq, Hkv, cap, seq_lens, scores, sstride, grid, pm, hist, s); break;
    case 2: launch_hamming_gr<2, R>(qc, kc, Hq, Hkv, cap, seq_lens, scores, sstride, grid, pm, hist, s); break;
    case 4: launch_hamming_gr<4, R>(qc, kc, Hq, Hkv, cap, seq_lens, scores, sstride, grid, pm, hist, s); break;
    case 8: launch_hamming_gr<8, R>(qc, kc, Hq, Hkv, cap, seq_lens, scores, sstride, grid, pm, hist, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_hamming(const uint32_t* qc, const uint32_t* kc, int B, int Hq, int Hkv,
                          int64_t cap, const int32_t* seq_lens, int64_t max_len, uint16_t* scores,
                          int64_t sstride, hipStream_t s, int r, const PageMap* pm, uint32_t* hist) {
  const int G = Hq / Hkv;
  const int64_t per_block = (int64_t)kNT * kHamTPT;
  dim3 grid((unsigned)((max_len + per_block - 1) / per_block), (unsigned)(B * Hkv));
  switch (r) {
    case 32: return launch_hamming_r<32>(qc, kc, G, Hq, Hkv, cap, seq_lens, scores, sstride, grid, pm, hist, s);
    case 64: return launch_hamming_r<64>(qc, kc, G, Hq, Hkv, cap, seq_lens, scores, sstride, grid, pm, hist, s);
    case 256: return launch_hamming_r<256>(qc, kc, G, Hq, Hkv, cap, seq_lens, scores, sstride, grid, pm, hist, s);
    default: return launch_hamming_r<128>(qc, kc, G, Hq, Hkv, cap, seq_lens, scores, sstride, grid, pm, hist, s);
  }
}

hipError_t launch_topk(const uint16_t* scores, int64_t sstride, int B, int Hkv, int64_t cap,
                       const int32_t* seq_lens, int k, int max_score, int32_t* idx, hipStream_t s,
                       void* scratch, int64_t max_len) {
  if (max_score + 1 > kMaxBins) return hipErrorInvalidValue;
  if (max_len > sstride) max_len = sstride;
  if (!scratch || max_len <= kTkChunk) {
    hipLaunchKernelGGL(topk_kernel, dim3(B * Hkv), dim3(kTopkNT), 0, s, scores, sstride, Hkv, cap,
                       seq_lens, k, max_score, idx);
    return hipGetLastError();
  }
  const int U = B * Hkv, nb = max_score + 1;
  const int chunks = (int)((max_len + kTkChunk - 1) / kTkChunk);
  uint32_t* hist = static_cast<uint32_t*>(scratch);
  uint32_t* params = hist + (size_t)U * nb;
  uint32_t* cnt = params + (size_t)U * 2;
  hipError_t e = launch_fill_zero(hist, (size_t)U * nb * 4, s);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)chunks, (unsigned)U);
  hipLaunchKernelGGL(topk_hist_kernel, grid, dim3(kNT), 0, s, scores, sstride, Hkv, cap, seq_lens, max_score, hist);
  hipLaunchKernelGGL(topk_thresh_kernel, dim3(U), dim3(kNT), 0, s, hist, nb, Hkv, cap, sstride, seq_lens, k, params,
                     idx);
  hipLaunchKernelGGL(topk_count_kernel, grid, dim3(kNT), 0, s, scores, sstride, Hkv, cap, seq_lens, max_score,
                     params, chunks, cnt, (const uint32_t*)hist, k, 0, idx);
  hipLaunchKernelGGL(topk_compact_kernel, grid, dim3(kNT), 0, s, scores, sstride, Hkv, cap, seq_lens, max_score,
                     (const uint32_t*)params, chunks, (const uint32_t*)cnt, k, idx);
  return hipGetLastError();
}

hipError_t launch_topk_after_hamming(const uint16_t* scores, int64_t sstride, int B, int Hkv, int64_t cap,
                                     const int32_t* seq_lens, int k, int max_score, int32_t* idx, hipStream_t s,
                                     void* scratch, int64_t max_len) {
  if (max_score + 1 > kMaxBins) return hipErrorInvalidValue;
  if (max_len > sstride) max_len = sstride;
  const int U = B * Hkv, nb = max_score + 1;
  const int chunks = (int)((max_len + kTkChunk - 1) / kTkChunk);
  const uint32_t* hist = static_cast<const uint32_t*>(scratch);
  uint32_t* params = static_cast<uint32_t*>(scratch) + (size_t)U * nb;
  uint32_t* cnt = params + (size_t)U * 2;
  const dim3 grid((unsigned)chunks, (unsigned)U);
  hipLaunchKernelGGL(topk_count_kernel, grid, dim3(kNT), 0, s, scores, sstride, Hkv, cap, seq_lens, max_score,
                     params, chunks, cnt, hist, k, 1, idx);
  hipLaunchKernelGGL(topk_compact_kernel, grid, dim3(kNT), 0, s, scores, sstride, Hkv, cap, seq_lens, max_score,
                     (const uint32_t*)params, chunks, (const uint32_t*)cnt, k, idx);
  return hipGetLastError();
}

}  // namespace hata
