// decode_step.hip -- the whole HATA decode step in one launch.
//
// HATA paper notes, section "Key design: Decode-stage algorithm" (encode the
// new query and key, append the key code, Hamming scores bitcount(xor),
// GQA aggregation, top-k, gather, sparse attention) and section
// "Hardware-efficient optimisation" (fused encode + cache update, XOR/popcount
// scoring with coalesced loads, gather fused into the attention kernel).
//
// Work split.  A unit is one (sequence b, KV head h).  Each unit owns Wg
// workgroups (co-resident: the host keeps units x Wg <= CU count); workgroup
// w owns tokens [w*chunk, (w+1)*chunk).  When the unit count is a multiple of
// 8 the block -> unit map keeps a unit's workgroups on one XCD (blocks are
// dealt round-robin over the 8 XCDs), so their exchanges stay XCD-local.
//
// Per workgroup:
//   1. issue the streaming loads of its code-cache rows (16 bytes per token);
//   2. encode the G query rows (and, for the owner of row n-1, the new key,
//      which is written to the cache): W_H columns in registers, two wave64
//      ballots per 128-bit code;
//   3. score every owned token with the bit-sliced GQA Hamming sum, keep the
//      scores in LDS and build an LDS histogram over [0, G*r];
//   4. publish a window of the histogram -- bins from its smallest score up
//      to its own k-th smallest (all of its bins when it has fewer than k
//      tokens) -- and wait for the unit's other workgroups.  The global
//      threshold T (smallest s with count(score <= s) >= k) cannot exceed any
//      workgroup's own k-th smallest score, so these windows determine T, the
//      count below T, and how many tied-at-T tokens each earlier workgroup
//      keeps (ties go to lower token indices, i.e. earlier workgroups first);
//   5. compact its kept tokens in index order (idx_out if requested);
//   6. attend its kept rows (gather-fused online softmax over G heads);
//   7. publish its (max, sum, acc) record per head, wait for the unit, and
//      merge a slice of the unit's outputs by log-sum-exp in fixed order.
// With Wg == 1 steps 4 and 7 need no exchange.
//
// Exchanges between workgroups use agent-coherent stores/loads into their
// own slots plus one monotonically increasing flag per workgroup; there is
// no same-address read-modify-write (those serialise at the memory side).
// Every wait is bounded; a timeout sets bit 0 of the workspace error word.
#include "hata_device.hpp"
#include "hata_launch.hpp"

namespace hata {

namespace {

constexpr int kMaxWg = 64;         // workgroups per unit (one polling wave)
constexpr int kWinWords = 64;      // 32-bit words per published window (128 uint16)
constexpr int kWinHdr = 8;         // uint16 header entries
constexpr int kWinCap = 2 * kWinWords - kWinHdr;  // histogram bins a window holds
constexpr int kMaxChunk = 32768;   // tokens per workgroup (uint16 scores in LDS)
constexpr int kPF = 16;            // code loads in flight per thread
constexpr uint32_t kSpinLimit = 1u << 22;

struct StepArgs {
  const uint16_t* q;
  const uint16_t* K;
  const uint16_t* V;
  const float* W;
  uint64_t* codes;
  const int32_t* seq_lens;
  float* out;
  int32_t* idx_out;
  int64_t cap;
  int Hq, Hkv, k;
  float scale;
  int Wg, chunk, xcd_map, U;
  uint32_t* err;
  uint32_t* flags;  // [U][kMaxWg]
  uint32_t* win;    // [U][kMaxWg][kWinWords]
  uint32_t* full;   // [U][kMaxWg][full_words]  (only for overflowing windows)
  float* part;      // [U][kMaxWg][G][kRec]
  int full_words;
};

template <int G>
struct Lds {
  static constexpr int NB = G * kR + 1;           // histogram bins
  static constexpr int NBP = (NB + 63) / 64 * 64;
  static constexpr int RED = (kMergeFloats<G> > (G + 1) * kD) ? kMergeFloats<G> : (G + 1) * kD;
  // offsets in bytes
  static constexpr int o_hist = 0;                               // NBP uint32
  static constexpr int o_qf = o_hist + NBP * 4;                  // (G+1)*128 float
  static constexpr int o_red = o_qf + (G + 1) * kD * 4;          // RED float
  static constexpr int o_qcode = o_red + RED * 4;                // (G+1)*2 uint64
  static constexpr int o_misc = o_qcode + (G + 1) * 16;          // 64 uint32
  static constexpr int o_wlt = o_misc + 64 * 4;                  // kMaxWg uint32
  static constexpr int o_weq = o_wlt + kMaxWg * 4;               // kMaxWg uint32
  static constexpr int o_win = o_weq + kMaxWg * 4;               // kMaxWg*kWinWords uint32
  static constexpr int o_sel = o_win + kMaxWg * kWinWords * 4;   // k int32
  static constexpr int fixed = o_sel;
  static size_t bytes(int k, int chunk) {
    size_t s = (size_t)fixed + (size_t)k * 4;
    s = (s + 15) / 16 * 16;
    return s + (size_t)chunk * 2;
  }
};

__device__ __forceinline__ void map_block(const StepArgs& a, int* unit, int* w) {
  const int bid = blockIdx.x;
  if (a.xcd_map) {
    const int xcd = bid & 7, slot = bid >> 3;
    const int uix = slot / a.Wg;
    *w = slot - uix * a.Wg;
    *unit = uix * 8 + xcd;
  } else {
    *unit = bid / a.Wg;
    *w = bid - *unit * a.Wg;
  }
}

// Wave 0 waits until every flag of the unit has reached `target`.
__device__ __forceinline__ void wait_unit(const StepArgs& a, int unit, uint32_t target) {
  const int lane = threadIdx.x & 63;
  if ((threadIdx.x >> 6) == 0) {
    const uint32_t* f = a.flags + (int64_t)unit * kMaxWg;
    uint32_t it = 0;
    while (true) {
      const uint32_t v = (lane < a.Wg) ? ld_agent(f + lane) : target;
      const bool ok = (int32_t)(v - target) >= 0;
      if (__all(ok)) break;
      if (++it > kSpinLimit) {
        if (lane == 0) atomicOr(a.err, 1u);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __syncthreads();
}

// In-place inclusive scan of hist[0, nb) with 256 threads; returns nothing,
// leaves cum in hist.  Also accumulates three counts into misc[0..2]:
// #bins with cum == 0, #bins with cum < cnt, #bins with cum < k.
template <int NB>
__device__ __forceinline__ void cum_hist(uint32_t* hist, uint32_t* misc, uint32_t* tmp, uint32_t cnt,
                                         uint32_t k) {
  constexpr int BPT = (NB + kNT - 1) / kNT;
  const int t = threadIdx.x;
  uint32_t v[BPT];
  uint32_t loc = 0;
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    const int s = t * BPT + j;
    v[j] = (s < NB) ? hist[s] : 0u;
    loc += v[j];
  }
  uint32_t tot;
  uint32_t run = block_excl_scan_u32(loc, tmp, &tot);
  uint32_t zero = 0, below_cnt = 0, below_k = 0;
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    const int s = t * BPT + j;
    if (s < NB) {
      run += v[j];
      hist[s] = run;
      zero += (run == 0);
      below_cnt += (run < cnt);
      below_k += (run < k);
    }
  }
  if (zero) atomicAdd(&misc[0], zero);
  if (below_cnt) atomicAdd(&misc[1], below_cnt);
  if (below_k) atomicAdd(&misc[2], below_k);
  __syncthreads();
}

template <int G>
__global__ __launch_bounds__(kNT) void decode_step_kernel(const StepArgs a) {
  using L = Lds<G>;
  constexpr int NB = L::NB;
  extern __shared__ __align__(16) unsigned char smem[];
  uint32_t* hist = reinterpret_cast<uint32_t*>(smem + L::o_hist);
  float* qf = reinterpret_cast<float*>(smem + L::o_qf);
  float* red = reinterpret_cast<float*>(smem + L::o_red);
  uint64_t* qcode = reinterpret_cast<uint64_t*>(smem + L::o_qcode);
  uint32_t* misc = reinterpret_cast<uint32_t*>(smem + L::o_misc);
  uint32_t* wlt = reinterpret_cast<uint32_t*>(smem + L::o_wlt);
  uint32_t* weq = reinterpret_cast<uint32_t*>(smem + L::o_weq);
  uint32_t* winl = reinterpret_cast<uint32_t*>(smem + L::o_win);
  int32_t* sel = reinterpret_cast<int32_t*>(smem + L::o_sel);
  uint16_t* sc = reinterpret_cast<uint16_t*>(smem + ((L::o_sel + a.k * 4 + 15) / 16 * 16));

  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  int unit, w;
  map_block(a, &unit, &w);
  const int b = unit / a.Hkv, h = unit - b * a.Hkv;
  const int64_t cap = a.cap;
  const int k = a.k;
  const int n = a.seq_lens[b];
  if (n < 1 || (int64_t)n > cap) {
    // invalid length: every workgroup of the unit leaves here, so the unit's
    // flags stay consistent; workgroup 0 clears the outputs
    if (w == 0) {
      for (int e = t; e < G * kD; e += kNT)
        a.out[((int64_t)b * a.Hq + (int64_t)h * G) * kD + e] = 0.f;
      if (a.idx_out)
        for (int j = t; j < k; j += kNT) a.idx_out[(int64_t)unit * k + j] = -1;
    }
    return;
  }
  const int64_t row0 = ((int64_t)b * a.Hkv + h) * cap;
  const int lo = w * a.chunk;
  const int cnt = max(0, min(n, lo + a.chunk) - lo);
  const bool owns_new = (n - 1 >= lo) && (n - 1 < lo + cnt);
  const int new_li = n - 1 - lo;

  uint32_t epoch = 0;
  if (a.Wg > 1 && wv == 0) epoch = ld_agent(a.flags + (int64_t)unit * kMaxWg + w);

  // ---- 1. first group of code-cache loads
  const uint4* cbase = reinterpret_cast<const uint4*>(a.codes) + row0 + lo;
  uint4 cbuf[kPF];
#pragma unroll
  for (int j = 0; j < kPF; ++j) {
    const int li = j * kNT + t;
    cbuf[j] = make_uint4(0, 0, 0, 0);
    if (li < cnt) cbuf[j] = load_stream16(cbase + li);
  }

  // ---- 2. encode q rows (+ new key row)
  const int col = (wv & 1) * 64 + lane, dh = wv >> 1;
  const float* Wh = a.W + (int64_t)h * kD * kR;
  float wr[64];
#pragma unroll
  for (int i = 0; i < 64; ++i) wr[i] = Wh[(dh * 64 + i) * kR + col];
  const int nrows = G + (owns_new ? 1 : 0);
  for (int e = t; e < nrows * 64; e += kNT) {
    const int r = e >> 6, c2 = e & 63;
    const uint32_t* src = (r < G)
        ? reinterpret_cast<const uint32_t*>(a.q + ((int64_t)b * a.Hq + (int64_t)h * G + r) * kD)
        : reinterpret_cast<const uint32_t*>(a.K + (row0 + n - 1) * kD);
    const uint32_t two = src[c2];
    qf[r * kD + 2 * c2] = bf16_lo(two);
    qf[r * kD + 2 * c2 + 1] = bf16_hi(two);
  }
  for (int i = t; i < L::NBP; i += kNT) hist[i] = 0;
  if (t < 64) misc[t] = 0;
  __syncthreads();
  float p[G + 1];
#pragma unroll
  for (int r = 0; r <= G; ++r) {
    float s = 0.f;
    if (r < nrows) {
#pragma unroll
      for (int i = 0; i < 64; ++i) s = fmaf(qf[r * kD + dh * 64 + i], wr[i], s);
    }
    p[r] = s;
  }
  if (dh == 1) {
#pragma unroll
    for (int r = 0; r <= G; ++r)
      if (r < nrows) red[r * kD + col] = p[r];
  }
  __syncthreads();
  if (dh == 0) {
#pragma unroll
    for (int r = 0; r <= G; ++r) {
      if (r < nrows) {
        const float s = p[r] + red[r * kD + col];
        const uint64_t m = __ballot(s >= 0.0f);
        if (lane == 0) qcode[r * 2 + (wv & 1)] = m;
      }
    }
  }
  __syncthreads();
  uint4 newc = make_uint4(0, 0, 0, 0);
  if (owns_new) {
    const uint64_t k0 = qcode[G * 2], k1 = qcode[G * 2 + 1];
    newc = make_uint4((uint32_t)k0, (uint32_t)(k0 >> 32), (uint32_t)k1, (uint32_t)(k1 >> 32));
    if (t == 0) reinterpret_cast<uint4*>(a.codes)[row0 + n - 1] = newc;
  }
  uint32_t qw[G][kWords32];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const uint64_t x0 = qcode[g * 2], x1 = qcode[g * 2 + 1];
    qw[g][0] = (uint32_t)x0; qw[g][1] = (uint32_t)(x0 >> 32);
    qw[g][2] = (uint32_t)x1; qw[g][3] = (uint32_t)(x1 >> 32);
  }
  QMasks<G> qm;
  build_qmasks<G>(qw, qm);

  // ---- 3. score the owned tokens
  for (int base = 0; base < cnt; base += kPF * kNT) {
    uint4 nbuf[kPF];
    const int nbase = base + kPF * kNT;
#pragma unroll
    for (int j = 0; j < kPF; ++j) {
      const int li = nbase + j * kNT + t;
      nbuf[j] = make_uint4(0, 0, 0, 0);
      if (li < cnt) nbuf[j] = load_stream16(cbase + li);
    }
#pragma unroll
    for (int j = 0; j < kPF; ++j) {
      const int li = base + j * kNT + t;
      if (li < cnt) {
        const uint4 c = (li == new_li) ? newc : cbuf[j];
        const uint32_t s = gqa_hamming<G>(c, qm);
        sc[li] = (uint16_t)s;
        atomicAdd(&hist[s], 1u);
      }
    }
#pragma unroll
    for (int j = 0; j < kPF; ++j) cbuf[j] = nbuf[j];
  }
  __syncthreads();

  // ---- 4. threshold
  cum_hist<NB>(hist, misc, misc + 8, (uint32_t)cnt, (uint32_t)k);
  // local stats: lo_w = first nonempty bin, hi_w = last nonempty bin,
  // tk = own k-th smallest score (if cnt >= k)
  const int lo_w = (int)misc[0];
  const int hi_w = (int)misc[1];
  const int tk = (int)misc[2];
  int T;
  uint32_t lt_all, quota, sel_before = 0, take_self;
  if (a.Wg == 1) {
    T = (cnt >= k) ? tk : NB - 1;
    lt_all = T > 0 ? hist[T - 1] : 0u;
    quota = (uint32_t)k - lt_all;
    const uint32_t eq_self = hist[T] - lt_all;
    take_self = eq_self < quota ? eq_self : quota;
  } else {
    // publish the window [lo_w, top] of this workgroup's histogram
    const bool has_k = cnt >= k;
    const int top = (cnt == 0) ? -1 : (has_k ? tk : hi_w);
    const int wlo = (cnt == 0) ? 0 : lo_w;
    const int len = top - wlo + 1;
    const bool ovf = len > kWinCap;
    uint32_t* mywin = a.win + ((int64_t)unit * kMaxWg + w) * kWinWords;
    if (t < kWinWords) {
      uint32_t word;
      if (t < kWinHdr / 2) {
        const uint32_t hv[kWinHdr] = {(uint32_t)wlo, (uint32_t)(top + 1), has_k ? 1u : 0u,
                                      ovf ? 1u : 0u, (uint32_t)cnt & 0xFFFFu, (uint32_t)cnt >> 16,
                                      0u, 0u};
        word = hv[2 * t] | (hv[2 * t + 1] << 16);
      } else {
        uint32_t two[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int j = 2 * t + e - kWinHdr;
          const int s = wlo + j;
          uint32_t c = 0;
          if (j < len && j < kWinCap) c = hist[s] - (s > 0 ? hist[s - 1] : 0u);
          two[e] = c;
        }
        word = two[0] | (two[1] << 16);
      }
      st_agent(mywin + t, word);
    }
    if (ovf) {
      uint32_t* myfull = a.full + ((int64_t)unit * kMaxWg + w) * a.full_words;
      for (int i = t; i < a.full_words; i += kNT) {
        uint32_t two[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int s = 2 * i + e;
          two[e] = (s < NB) ? hist[s] - (s > 0 ? hist[s - 1] : 0u) : 0u;
        }
        st_agent(myfull + i, two[0] | (two[1] << 16));
      }
    }
    wait_all_mem();
    __syncthreads();
    if (t == 0) st_agent(a.flags + (int64_t)unit * kMaxWg + w, epoch + 1);
    wait_unit(a, unit, epoch + 1);

    // read every window of the unit
    const uint32_t* uwin = a.win + (int64_t)unit * kMaxWg * kWinWords;
    for (int i = t; i < a.Wg * kWinWords; i += kNT) winl[i] = ld_agent(uwin + i);
    __syncthreads();
    // bound on T: the smallest own-k-th score among workgroups that have one
    if (t < 16) misc[t] = 0;
    __syncthreads();
    if (t < a.Wg) {
      const uint32_t h0 = winl[t * kWinWords], h1 = winl[t * kWinWords + 1];
      const bool whas = (h1 & 0xFFFFu) != 0;
      const int wtop = (int)(h0 >> 16) - 1;
      if (whas) atomicMax(&misc[4], (uint32_t)(NB - wtop));  // NB - (min top)
    }
    __syncthreads();
    const int tmin = misc[4] ? NB - (int)misc[4] : NB - 1;
    // global histogram over [0, tmin]
    for (int i = t; i < L::NBP; i += kNT) hist[i] = 0;
    __syncthreads();
    for (int ww = 0; ww < a.Wg; ++ww) {
      const uint32_t* wr16 = winl + ww * kWinWords;
      const uint32_t h0 = wr16[0], h1 = wr16[1];
      const int wlo2 = min((int)(h0 & 0xFFFF), NB);
      const int wtop = min((int)(h0 >> 16) - 1, NB - 1);
      const bool wovf = (h1 >> 16) & 1u;
      int hi2 = min(wtop, tmin);
      if (!wovf) {
        hi2 = min(hi2, wlo2 + kWinCap - 1);
        for (int s = wlo2 + t; s <= hi2; s += kNT) {
          const int j = s - wlo2 + kWinHdr;
          const uint32_t c = (wr16[j >> 1] >> ((j & 1) * 16)) & 0xFFFFu;
          if (c) atomicAdd(&hist[s], c);
        }
      } else {
        const uint32_t* wf = a.full + ((int64_t)unit * kMaxWg + ww) * a.full_words;
        for (int s = wlo2 + t; s <= hi2; s += kNT) {
          const uint32_t c = (ld_agent(wf + (s >> 1)) >> ((s & 1) * 16)) & 0xFFFFu;
          if (c) atomicAdd(&hist[s], c);
        }
      }
    }
    if (t < 16) misc[t] = 0;
    __syncthreads();
    cum_hist<NB>(hist, misc, misc + 8, 0xFFFFFFFFu, (uint32_t)k);
    // bins beyond tmin hold cum == C(tmin); T = #bins with C < k, capped at tmin
    T = (int)misc[2];
    if (T > tmin) T = tmin;
    lt_all = T > 0 ? hist[T - 1] : 0u;
    quota = (uint32_t)k - lt_all;
    // per-workgroup counts below and at T
    if (t < a.Wg) {
      const uint32_t* wr16 = winl + t * kWinWords;
      const uint32_t h0 = wr16[0], h1 = wr16[1];
      const int wlo2 = min((int)(h0 & 0xFFFF), NB);
      const int wtop = min((int)(h0 >> 16) - 1, NB - 1);
      const bool wovf = (h1 >> 16) & 1u;
      const uint32_t* wf = a.full + ((int64_t)unit * kMaxWg + t) * a.full_words;
      uint32_t lt = 0, eq = 0;
      const int last = wovf ? min(wtop, T) : min(min(wtop, T), wlo2 + kWinCap - 1);
      for (int s = wlo2; s <= last; ++s) {
        uint32_t c;
        if (!wovf) {
          const int j = s - wlo2 + kWinHdr;
          c = (wr16[j >> 1] >> ((j & 1) * 16)) & 0xFFFFu;
        } else {
          c = (ld_agent(wf + (s >> 1)) >> ((s & 1) * 16)) & 0xFFFFu;
        }
        if (s < T) lt += c; else eq += c;
      }
      wlt[t] = lt;
      weq[t] = eq;
    }
    __syncthreads();
    uint32_t pre_lt = 0, pre_eq = 0;
    for (int ww = 0; ww < w; ++ww) { pre_lt += wlt[ww]; pre_eq += weq[ww]; }
    const uint32_t eq_self = weq[w];
    const uint32_t left = quota > pre_eq ? quota - pre_eq : 0u;
    take_self = eq_self < left ? eq_self : left;
    sel_before = pre_lt + (pre_eq < quota ? pre_eq : quota);
  }

  // ---- 5. ordered compaction of the kept tokens
  const int per = (cnt + kNT - 1) / kNT;
  const int i_begin = min(cnt, t * per), i_end = min(cnt, i_begin + per);
  uint32_t lt = 0, eq = 0;
  for (int i = i_begin; i < i_end; ++i) {
    const int s = sc[i];
    lt += (s < T);
    eq += (s == T);
  }
  uint32_t tot_lt, tot_eq;
  uint32_t lt_before = block_excl_scan_u32(lt, misc + 8, &tot_lt);
  uint32_t eq_before = block_excl_scan_u32(eq, misc + 12, &tot_eq);
  int32_t* idx_unit = a.idx_out ? a.idx_out + (int64_t)unit * k : nullptr;
  for (int i = i_begin; i < i_end; ++i) {
    const int s = sc[i];
    int pos = -1;
    if (s < T) {
      pos = (int)(lt_before + min(eq_before, take_self));
      ++lt_before;
    } else if (s == T) {
      if (eq_before < take_self) pos = (int)(lt_before + eq_before);
      ++eq_before;
    }
    // pos < m_self <= k and sel_before + m_self <= min(k, n) by construction;
    // the bounds are re-checked so a broken invariant cannot write outside
    if (pos >= 0 && pos < k) {
      sel[pos] = lo + i;
      if (idx_unit && sel_before + (uint32_t)pos < (uint32_t)k) idx_unit[sel_before + pos] = lo + i;
    }
  }
  if (idx_unit && w == 0)
    for (int j = min(k, n) + t; j < k; j += kNT) idx_unit[j] = -1;
  const int m_self = min(k, (int)(tot_lt + min(tot_eq, take_self)));
  __syncthreads();

  // ---- 6. gather-fused attention over the kept rows
  const int slot = t >> 4, sub = t & 15;
  float qreg[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int c = 0; c < 8; ++c) qreg[g][c] = qf[g * kD + sub * 8 + c];
  const uint16_t* Kb = a.K + row0 * kD + sub * 8;
  const uint16_t* Vb = a.V + row0 * kD + sub * 8;
  SoftmaxState<G> st;
  st.init();
  constexpr int UN = 2;
  for (int r0 = slot; r0 < m_self; r0 += 16 * UN) {
    uint4 kv[UN], vv[UN];
    bool valid[UN];
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int r = r0 + 16 * u;
      valid[u] = r < m_self;
      kv[u] = make_uint4(0, 0, 0, 0);
      vv[u] = make_uint4(0, 0, 0, 0);
      if (valid[u]) {
        const int64_t tok = min(max(sel[r], 0), n - 1);
        kv[u] = *reinterpret_cast<const uint4*>(Kb + tok * kD);
        vv[u] = *reinterpret_cast<const uint4*>(Vb + tok * kD);
      }
    }
    attend_block<G, UN>(st, qreg, kv, vv, valid, a.scale);
  }
  merge_wg<G>(st, red);

  float* outp = a.out + ((int64_t)b * a.Hq + (int64_t)h * G) * kD;
  if (a.Wg == 1) {
    for (int e = t; e < G * kD; e += kNT) {
      const int g = e / kD, c = e % kD;
      const float* r = red + g * kRec;
      outp[e] = (r[1] > 0.f) ? r[2 + c] / r[1] : 0.f;
    }
    return;
  }

  // ---- 7. publish this workgroup's records, wait, merge a slice
  float* mypart = a.part + ((int64_t)unit * kMaxWg + w) * (G * kRec);
  for (int e = t; e < G * kRec; e += kNT) st_agent(mypart + e, red[e]);
  wait_all_mem();
  __syncthreads();
  if (t == 0) st_agent(a.flags + (int64_t)unit * kMaxWg + w, epoch + 2);
  wait_unit(a, unit, epoch + 2);
  const int per_wg = (G * kD + a.Wg - 1) / a.Wg;
  const int e0 = w * per_wg, e1 = min(G * kD, e0 + per_wg);
  const float* upart = a.part + (int64_t)unit * kMaxWg * (G * kRec);
  for (int e = e0 + t; e < e1; e += kNT) {
    const int g = e / kD, c = e % kD;
    float M = -INFINITY;
    for (int ww = 0; ww < a.Wg; ++ww) M = fmaxf(M, ld_agent(upart + ww * (G * kRec) + g * kRec));
    float Ls = 0.f, A = 0.f;
    if (M != -INFINITY) {
      for (int ww = 0; ww < a.Wg; ++ww) {
        const float* r = upart + ww * (G * kRec) + g * kRec;
        const float f = __expf(ld_agent(r) - M);
        Ls = fmaf(ld_agent(r + 1), f, Ls);
        A = fmaf(ld_agent(r + 2 + c), f, A);
      }
    }
    outp[e] = (Ls > 0.f) ? A / Ls : 0.f;
  }
  // keep every flag slot of the unit equal for the next launch (which may
  // use a different number of workgroups per unit)
  if (w == 0 && t >= a.Wg && t < kMaxWg)
    st_agent(a.flags + (int64_t)unit * kMaxWg + t, epoch + 2);
}

}  // namespace

StepPlan plan_decode_step(int B, int Hq, int Hkv, int64_t max_len, int k, int num_cus) {
  StepPlan p;
  p.G = Hq / Hkv;
  p.U = B * Hkv;
  const int U = p.U;
  int Wg = num_cus / (U > 0 ? U : 1);
  if (Wg < 1) Wg = 1;
  if (Wg > kMaxWg) Wg = kMaxWg;
  const int64_t by_tokens = (max_len + kNT - 1) / kNT;  // at least 256 tokens per workgroup
  if (Wg > by_tokens) Wg = (int)(by_tokens < 1 ? 1 : by_tokens);
  int64_t chunk = (max_len + Wg - 1) / Wg;
  chunk = (chunk + kNT - 1) / kNT * kNT;
  p.fused = true;
  if (chunk > kMaxChunk) {
    const int64_t need = (max_len + kMaxChunk - 1) / kMaxChunk;
    if (need > kMaxWg || (int64_t)U * need > num_cus) {
      p.fused = false;
    } else {
      Wg = (int)need;
      chunk = (max_len + Wg - 1) / Wg;
      chunk = (chunk + kNT - 1) / kNT * kNT;
    }
  }
  p.Wg = Wg;
  p.chunk = (int)chunk;
  p.xcd_map = (Wg > 1 && U % 8 == 0) ? 1 : 0;
  auto align = [](size_t x) { return (x + 255) / 256 * 256; };
  const int G = p.G;
  const int NB = G * kR + 1;
  p.full_words = (NB + 1) / 2;
  size_t off = 0;
  p.off_err = off;   off = align(off + 256);
  if (p.fused) {
    switch (G) {
      case 1: p.lds_bytes = Lds<1>::bytes(k, p.chunk); break;
      case 2: p.lds_bytes = Lds<2>::bytes(k, p.chunk); break;
      case 4: p.lds_bytes = Lds<4>::bytes(k, p.chunk); break;
      default: p.lds_bytes = Lds<8>::bytes(k, p.chunk); break;
    }
    const size_t slots = (size_t)U * kMaxWg;
    p.off_flags = off; off = align(off + slots * 4);
    if (Wg > 1) {
      p.off_win = off;  off = align(off + slots * kWinWords * 4);
      p.off_full = off; off = align(off + slots * (size_t)p.full_words * 4);
      p.off_part = off; off = align(off + slots * (size_t)G * kRec * 4);
    }
  } else {
    // staged steps inside hata_decode_step
    p.off_qc = off;     off = align(off + (size_t)B * Hq * 16);
    p.off_scores = off; off = align(off + (size_t)U * max_len * 2);
    p.off_attn = off;   off = align(off + attn_part_floats(B, Hkv, G, k) * 4);
  }
  p.total = off;
  return p;
}

template <int G>
static hipError_t launch_step_g(const StepPlan& p, const StepArgs& a, hipStream_t s) {
  const size_t lds = p.lds_bytes;
  static bool configured = false;  // raise the dynamic-LDS limit once per instantiation
  if (!configured) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_step_kernel<G>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    configured = true;
  }
  hipLaunchKernelGGL(decode_step_kernel<G>, dim3(p.U * p.Wg), dim3(kNT), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_decode_step(const StepPlan& p, const uint16_t* q, const uint16_t* K,
                              const uint16_t* V, const float* W, uint64_t* codes, int B, int Hq,
                              int Hkv, int64_t cap, const int32_t* seq_lens, int k, float scale,
                              float* out, int32_t* idx_out, unsigned char* ws, hipStream_t s) {
  StepArgs a;
  a.q = q; a.K = K; a.V = V; a.W = W; a.codes = codes; a.seq_lens = seq_lens;
  a.out = out; a.idx_out = idx_out; a.cap = cap; a.Hq = Hq; a.Hkv = Hkv; a.k = k;
  a.scale = scale; a.Wg = p.Wg; a.chunk = p.chunk; a.xcd_map = p.xcd_map; a.U = p.U;
  a.err = reinterpret_cast<uint32_t*>(ws + p.off_err);
  a.flags = reinterpret_cast<uint32_t*>(ws + p.off_flags);
  a.win = p.Wg > 1 ? reinterpret_cast<uint32_t*>(ws + p.off_win) : nullptr;
  a.full = p.Wg > 1 ? reinterpret_cast<uint32_t*>(ws + p.off_full) : nullptr;
  a.part = p.Wg > 1 ? reinterpret_cast<float*>(ws + p.off_part) : nullptr;
  a.full_words = p.full_words;
  (void)B;
  switch (p.G) {
    case 1: return launch_step_g<1>(p, a, s);
    case 2: return launch_step_g<2>(p, a, s);
    case 4: return launch_step_g<4>(p, a, s);
    case 8: return launch_step_g<8>(p, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace hata
