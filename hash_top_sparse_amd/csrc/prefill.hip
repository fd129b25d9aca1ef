// prefill.hip -- causal prefill attention on the matrix cores, with the key
// codes formed while each key tile sits in LDS.
//
// HATA notes, section "Method", "Overall framework", second stage: during
// prefill, attention is computed as usual while the keys are encoded into
// binary hash codes and cached; section "Key findings": the encode adds
// under one percent to prefill compute because r is far below the sequence
// length.  Here the encode reuses the key tile that the attention has
// already staged in LDS, so the keys are read from HBM once for both.
//
// Work split: one workgroup per (sequence, KV head, block of 128 query rows)
// where the 128 rows are the G query heads of the KV head times 128/G
// positions, so the G heads share every staged K/V tile.  Wave w owns 32
// (head, position) pairs.  Per 64-key tile:
//   S^T = K Q^T   v_mfma_f32_32x32x16_bf16, A = K rows from LDS, B = this
//                 wave's queries (registers); a lane's accumulators all
//                 belong to one query (lane % 32), half its keys each in
//                 lanes l and l ^ 32
//   online softmax in the log2 domain (scale * log2 e folded into the
//                 logits), row max / sum over the lane pair; the running
//                 sums are rescaled only when a row's max passes the
//                 reference by more than 2^8 in weight
//   O^T += V^T P^T  A = V^T from a transposed LDS copy, B = P rounded to
//                 bf16 straight from the S^T accumulators; the MFMA's k
//                 index runs over the keys in the order the accumulators
//                 hold them (any order gives the same contraction as long as
//                 A and B agree)
// The workgroup also encodes its own rows [p0, p0 + 128/G): when a tile
// holding some of them is staged, each wave multiplies the 32-row halves of
// the tile by 32-column slices of W_H split into two bf16 terms, in the same
// order of products and accumulations as the bulk encode (so the codes are
// the same bit for bit), takes the sign with ballots and collects the 32-bit
// code words in LDS; the rows go to the cache at the end.
//
// Blocks are issued heaviest first (the causal work grows with the position)
// and (sequence, KV head) varies fastest, so with B * Hkv a multiple of 8
// each XCD serves whole heads and their K/V stay in its L2.
#include "hata_device.hpp"
#include "hata_launch.hpp"

namespace hata {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBK = 64;              // keys per staged tile
constexpr float kLazyLog2 = 8.f;     // reference-max slack (log2 units)
constexpr int kKsStride = kD + 8;    // bf16 per staged key row (272 bytes)
constexpr int kVtStride = kBK + 4;   // bf16 per transposed value row (136 bytes)
constexpr int kBufElems = kBK * kKsStride + kD * kVtStride;  // bf16 per K/V tile buffer

template <int G, int R>
constexpr size_t prefill_lds_bytes() {
  return 2 * kBufElems * sizeof(uint16_t) + (128 / G) * (R / 32) * sizeof(uint32_t);
}

struct PrefillArgs {
  const uint16_t* q;
  const uint16_t* K;
  const uint16_t* V;
  const float* W;
  uint32_t* codes;  // rows of R/32 32-bit words
  const int32_t* seq_lens;
  float* out;
  int B, Hq, Hkv;
  int64_t q_rows, cap;
  int max_len, nqb;
  float scale_log2;
  PageMap pm;  // PAGED: K, V and codes are page pools addressed through it
};

// PAGED: K, V and codes are page pools (a.pm); a separate instance, the
// contiguous code is unchanged.
template <int G, int R, bool PAGED>
__global__ __launch_bounds__(kNT, 2) void prefill_kernel(PrefillArgs a) {
  constexpr int QP = 128 / G;         // positions per workgroup
  constexpr int CT = R / 32;          // 32-column slices of the code
  // two K/V tile buffers (the next tile is stored while the current one is
  // multiplied: one barrier per tile), then the code words
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* lds = reinterpret_cast<uint16_t*>(smem);
  uint32_t* cw = reinterpret_cast<uint32_t*>(smem + 2 * kBufElems * sizeof(uint16_t));

  const int t = threadIdx.x, lane = t & 63, half = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(t >> 6);
  const int heads = a.B * a.Hkv;
  const int bh = blockIdx.x % heads;
  const int qb = a.nqb - 1 - (int)(blockIdx.x / heads);
  const int b = bh / a.Hkv, hk = bh - b * a.Hkv;
  const int p0 = qb * QP;
  const int L = min(max(a.seq_lens[b], 0), a.max_len);
  if (p0 >= L) return;
  const int pend = min(p0 + QP, L);
  const int ntiles = (pend + kBK - 1) / kBK;

  // this lane's query: pair 32 wv + lane % 32 -> (head, position)
  const int pair = 32 * wv + (lane & 31);
  const int hq = hk * G + pair / QP;
  const int pos = p0 + pair % QP;
  const bool qvalid = pos < L;
  const int wpos_min = p0 + (32 * wv) % QP;
  const int wpos_max = min(wpos_min + (QP < 32 ? QP : 32) - 1, L - 1);
  const bool wactive = wpos_min < L;

  bf16x8 qf[8];
  {
    const uint16_t* qrow = a.q + (((int64_t)b * a.Hq + hq) * a.q_rows + (qvalid ? pos : 0)) * kD;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (qvalid) v = *reinterpret_cast<const uint4*>(qrow + 16 * s + 8 * half);
      qf[s] = __builtin_bit_cast(bf16x8, v);
    }
  }

  const int64_t kvoff = ((int64_t)b * a.Hkv + hk) * a.cap * kD;
  const uint16_t* Kh = a.K + kvoff;
  const uint16_t* Vh = a.V + kvoff;
  uint4 kreg[4], vreg[4];
  // value staging: thread t loads rows 4 vkg .. 4 vkg + 3 at columns 8 vc ..
  // 8 vc + 7 and writes them transposed, 4 keys per 8-byte store.  A store
  // of element e lands at dword 34 (8 vc + e) + 2 vkg, i.e. bank
  // 16 vc + 34 e + 2 vkg (mod 64): with vkg = t % 16 and the two column
  // blocks of each half-wave 2 apart, the 32 lanes of a half-wave hit 32
  // distinct bank pairs.
  const int vkg = t & 15, vu = t >> 4;
  const int vc = 4 * (vu >> 2) + ((vu & 1) << 1) + ((vu >> 1) & 1);
  // element offsets inside a tile: key chunk i of this thread is row
  // t/16 + 16 i, columns 8 (t % 16) ..; value chunk i is row 4 vkg + i
  const int koff = (t >> 4) * kD + (t & 15) * 8;
  const int voff = 4 * vkg * kD + vc * 8;
  // PAGED: the page ids of the next tile to fetch, loaded one fetch ahead so
  // that a tile's loads do not wait for the block table (rows clamped below
  // L).  Pages of >= 64 rows hold whole tiles: one id per tile (tpg), and the
  // tile is then read like a contiguous one; smaller pages: the ids of this
  // thread's 4 key rows and 4 value rows.
  const bool whole = PAGED && a.pm.log2P >= 6;
  int tpg = 0, kpg[4] = {}, vpg[4] = {};
  auto load_pages = [&](int tile) {
    if (whole) {
      tpg = a.pm.page(b, tile * kBK);
      return;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kpg[i] = a.pm.page(b, min(tile * kBK + (t >> 4) + 16 * i, L - 1));
      vpg[i] = a.pm.page(b, min(tile * kBK + 4 * vkg + i, L - 1));
    }
  };
  if constexpr (PAGED) load_pages(0);
  auto fetch = [&](int tile) {
    const uint16_t* kt = Kh + (int64_t)tile * kBK * kD;
    const uint16_t* vtl = Vh + (int64_t)tile * kBK * kD;
    if constexpr (PAGED) {
      if (whole) {
        const int64_t base = a.pm.at(tpg, hk, a.Hkv, tile * kBK) * kD;
        kt = a.K + base;
        vtl = a.V + base;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kr = tile * kBK + (t >> 4) + 16 * i, vr = tile * kBK + 4 * vkg + i;
          kreg[i] = kr < L ? *reinterpret_cast<const uint4*>(a.K + a.pm.at(kpg[i], hk, a.Hkv, kr) * kD +
                                                             (t & 15) * 8)
                           : make_uint4(0, 0, 0, 0);
          vreg[i] = vr < L ? *reinterpret_cast<const uint4*>(a.V + a.pm.at(vpg[i], hk, a.Hkv, vr) * kD + vc * 8)
                           : make_uint4(0, 0, 0, 0);
        }
        if (tile + 1 < ntiles) load_pages(tile + 1);
        return;
      }
      if (tile + 1 < ntiles) load_pages(tile + 1);
    }
    if (tile * kBK + kBK <= L) {  // a full tile (all but possibly the last)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        kreg[i] = *reinterpret_cast<const uint4*>(kt + koff + i * 16 * kD);
        vreg[i] = *reinterpret_cast<const uint4*>(vtl + voff + i * kD);
      }
    } else {
      const int rows = L - tile * kBK;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        kreg[i] = (t >> 4) + 16 * i < rows ? *reinterpret_cast<const uint4*>(kt + koff + i * 16 * kD)
                                           : make_uint4(0, 0, 0, 0);
        vreg[i] = 4 * vkg + i < rows ? *reinterpret_cast<const uint4*>(vtl + voff + i * kD) : make_uint4(0, 0, 0, 0);
      }
    }
  };

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;

  const float* Wh = a.W + (int64_t)hk * kD * R;

  auto stage = [&](int buf) {
    uint16_t* ksb = lds + buf * kBufElems;
    uint16_t* vtb = ksb + kBK * kKsStride;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = t + kNT * i, key = id >> 4, c = id & 15;
      *reinterpret_cast<uint4*>(ksb + key * kKsStride + c * 8) = kreg[i];
    }
    // element e of four rows -> 4 keys of one column: one byte permute per
    // pair of rows (bytes 0-3 of the selector's source are the second
    // operand, 4-7 the first)
    const uint32_t w0[4] = {vreg[0].x, vreg[0].y, vreg[0].z, vreg[0].w};
    const uint32_t w1[4] = {vreg[1].x, vreg[1].y, vreg[1].z, vreg[1].w};
    const uint32_t w2[4] = {vreg[2].x, vreg[2].y, vreg[2].z, vreg[2].w};
    const uint32_t w3[4] = {vreg[3].x, vreg[3].y, vreg[3].z, vreg[3].w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      const uint32_t lo = __builtin_amdgcn_perm(w1[e >> 1], w0[e >> 1], sel);
      const uint32_t hi = __builtin_amdgcn_perm(w3[e >> 1], w2[e >> 1], sel);
      *reinterpret_cast<uint2*>(vtb + (vc * 8 + e) * kVtStride + 4 * vkg) = make_uint2(lo, hi);
    }
  };
  fetch(0);
  stage(0);
  if (ntiles > 1) fetch(1);
  for (int tile = 0; tile < ntiles; ++tile) {
    // tile's buffer is complete and every wave is done with the other
    // buffer (tile - 1): store tile + 1 there and fetch tile + 2
    __syncthreads();
    if (tile + 1 < ntiles) {
      stage((tile + 1) & 1);
      if (tile + 2 < ntiles) fetch(tile + 2);
    }
    const uint16_t* ks = lds + (tile & 1) * kBufElems;
    const uint16_t* vt = ks + kBK * kKsStride;
    const int k0 = tile * kBK;

    if (wactive && k0 <= wpos_max) {
      const bool act1 = k0 + 32 <= wpos_max;
      f32x16 s[2];
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[st][i] = 0.f;
      {
        // the two 32-key halves as two independent accumulation chains in
        // one block, so their MFMAs and fragment reads interleave
        const uint16_t* krow = ks + (lane & 31) * kKsStride + 8 * half;
        // raised wave priority while the logit MFMAs issue: the other
        // workgroup's wave on this SIMD, in its softmax, then yields issue
        // slots to them (9.17 -> 9.09 ms at 32K)
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(1);
        if (act1) {
#pragma unroll
          for (int kk = 0; kk < 8; ++kk) {
            const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(krow + 16 * kk);
            const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(krow + 32 * kKsStride + 16 * kk);
            s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[kk], s[0], 0, 0, 0);
            s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[kk], s[1], 0, 0, 0);
          }
        } else {
#pragma unroll
          for (int kk = 0; kk < 8; ++kk) {
            const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(krow + 16 * kk);
            s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[kk], s[0], 0, 0, 0);
          }
        }
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
      }
      // Online softmax and O^T += V^T P^T, one 32-key half at a time, so the
      // softmax of the first half overlaps the second half's score MFMAs
      // and the second half's softmax overlaps the first half's value
      // MFMAs.  Causal mask and running max on the raw scores (the scale is
      // positive, so it commutes with the max and is applied inside the
      // exponent: p = 2^(s c - m c)).
      const bool need_mask = k0 + kBK - 1 > wpos_min;  // some key may follow some query of the wave
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        if (st == 1 && !act1) continue;
        float mx = -INFINITY;
        if (need_mask) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = k0 + 32 * st + 8 * (i >> 2) + (i & 3) + 4 * half;
            if (key > pos) s[st][i] = -INFINITY;
            mx = fmaxf(mx, s[st][i]);
          }
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[st][i]);
        }
        mx = pair32_max(mx);
        // The weights are taken relative to a reference max m_run, which
        // moves only when some row's max has risen past it by more than
        // kLazyLog2 in the exponent (or on a row's first unmasked keys):
        // weights stay below 2^kLazyLog2, keep bf16's relative precision
        // when rounded, and the final division by the row sum removes the
        // reference.  When the wave moves it, every row takes its own
        // max(m_run, mx), rounded as before, so a row whose max did not rise
        // gets alpha = 1 exactly.
        const bool rise = __fmul_rn(mx, a.scale_log2) > __fmul_rn(m_run, a.scale_log2) + kLazyLog2;
        const bool move = __ballot(rise) != 0;
        const float m_ref = move ? fmaxf(m_run, mx) : m_run;
        const float mref = m_ref == -INFINITY ? 0.f : __fmul_rn(m_ref, a.scale_log2);
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[st][i], a.scale_log2, -mref));
          s[st][i] = p;
          psum += p;
        }
        if (move) {
          const float alpha = __builtin_amdgcn_exp2f(__fmul_rn(m_run, a.scale_log2) - mref);
          l_run *= alpha;
#pragma unroll
          for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;
        }
        l_run += psum;
        m_run = m_ref;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          bf16x8 pf;
#pragma unroll
          for (int j = 0; j < 8; ++j) pf[j] = (__bf16)s[st][8 * kk + j];
          const int key0 = 32 * st + 16 * kk + 4 * half;
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) {
            const uint16_t* vrow = vt + (32 * dt + (lane & 31)) * kVtStride + key0;
            const uint2 x0 = *reinterpret_cast<const uint2*>(vrow);
            const uint2 x1 = *reinterpret_cast<const uint2*>(vrow + 8);
            const bf16x8 vf = __builtin_bit_cast(bf16x8, make_uint4(x0.x, x0.y, x1.x, x1.y));
            o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, o[dt], 0, 0, 0);
          }
        }
      }
    }
  }

  // normalise and store this lane's query row: accumulator i of slice dt
  // holds column 32 dt + 8 (i/4) + i%4 + 4 half
  const float l_tot = pair32_sum(l_run);
  if (qvalid) {
    const float inv = 1.f / l_tot;
    float* orow = a.out + (((int64_t)b * a.Hq + hq) * a.q_rows + pos) * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 v = make_float4(o[dt][4 * g] * inv, o[dt][4 * g + 1] * inv, o[dt][4 * g + 2] * inv,
                                     o[dt][4 * g + 3] * inv);
        *reinterpret_cast<float4*>(orow + 32 * dt + 8 * g + 4 * half) = v;
      }
  }
  // encode this workgroup's own rows [p0, pend).  They lie in the last
  // staged tile, still in LDS, except for G = 1 (128 positions, two tiles),
  // where both tiles are staged again (from L2: they were read a moment
  // ago).  Done after the output store so the attention registers are free.
  const bool restage = ntiles - 1 != p0 / kBK;
  // the last tile's buffer, or buffer 0 for the restaged tiles
  uint16_t* ks = lds + (restage ? 0 : ((ntiles - 1) & 1) * kBufElems);
  for (int tile = p0 / kBK; tile < ntiles; ++tile) {
    const int k0 = tile * kBK;
    if (restage) {
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int id = t + kNT * i, key = id >> 4, c = id & 15;
        const int row = k0 + key;
        const int64_t at = PAGED ? a.pm.row(b, hk, a.Hkv, row) : (int64_t)row + kvoff / kD;
        const uint4 v = row < L ? *reinterpret_cast<const uint4*>(a.K + at * kD + c * 8) : make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4*>(ks + key * kKsStride + c * 8) = v;
      }
      __syncthreads();
    }
    {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int r0 = k0 + 32 * st;
        if (r0 >= pend || r0 + 31 < p0) continue;
        const uint16_t* krow = ks + (32 * st + (lane & 31)) * kKsStride + 8 * half;
        for (int ct = wv; ct < CT; ct += 4) {
          f32x16 e;
#pragma unroll
          for (int i = 0; i < 16; ++i) e[i] = 0.f;
#pragma unroll 1
          for (int kk = 0; kk < 8; ++kk) {
            bf16x8 w1, w2;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const float v = Wh[(16 * kk + 8 * half + j) * R + 32 * ct + (lane & 31)];
              const __bf16 a1 = (__bf16)v;
              w1[j] = a1;
              w2[j] = (__bf16)(v - (float)a1);
            }
            const bf16x8 af = *reinterpret_cast<const bf16x8*>(krow + 16 * kk);
            e = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, w1, e, 0, 0, 0);
            e = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, w2, e, 0, 0, 0);
          }
          // element i: lanes 0-31 hold row 8 (i/4) + i%4, lanes 32-63 the
          // row 4 below, at columns 32 ct + lane % 32
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const uint64_t m = __ballot(e[i] >= 0.0f);
            if (lane == 0) {
              const int key = r0 + 8 * (i >> 2) + (i & 3);
              if (key >= p0 && key < pend) cw[(key - p0) * CT + ct] = (uint32_t)m;
              if (key + 4 >= p0 && key + 4 < pend) cw[(key + 4 - p0) * CT + ct] = (uint32_t)(m >> 32);
            }
          }
        }
      }
    }
  }
  __syncthreads();

  // code rows [p0, pend): CT = R/32 words each
  uint32_t* crow = a.codes + (((int64_t)b * a.Hkv + hk) * a.cap + p0) * CT;
  for (int e = t; e < (pend - p0) * CT; e += kNT) {
    const int row = e / CT, w = e - row * CT;
    if constexpr (PAGED)
      a.codes[a.pm.row(b, hk, a.Hkv, p0 + row) * CT + w] = cw[e];
    else
      crow[e] = cw[e];
  }
}

template <int G, int R, bool PAGED>
hipError_t launch_gr(const PrefillArgs& a, hipStream_t s) {
  constexpr size_t lds = prefill_lds_bytes<G, R>();
  static bool configured = false;  // dynamic LDS above 64 KiB needs an opt-in per kernel
  if (!configured) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_kernel<G, R, PAGED>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    configured = true;
  }
  const dim3 grid((unsigned)((int64_t)a.nqb * a.B * a.Hkv));
  hipLaunchKernelGGL((prefill_kernel<G, R, PAGED>), grid, dim3(kNT), lds, s, a);
  return hipGetLastError();
}

template <int G, bool PAGED>
hipError_t launch_g(const PrefillArgs& a, int r, hipStream_t s) {
  switch (r) {
    case 32: return launch_gr<G, 32, PAGED>(a, s);
    case 64: return launch_gr<G, 64, PAGED>(a, s);
    case 128: return launch_gr<G, 128, PAGED>(a, s);
    case 256: return launch_gr<G, 256, PAGED>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <bool PAGED>
hipError_t launch_p(const PrefillArgs& a, int G, int r, hipStream_t s) {
  switch (G) {
    case 1: return launch_g<1, PAGED>(a, r, s);
    case 2: return launch_g<2, PAGED>(a, r, s);
    case 4: return launch_g<4, PAGED>(a, r, s);
    case 8: return launch_g<8, PAGED>(a, r, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int prefill_positions_per_block(int G) { return 128 / G; }

hipError_t launch_prefill(const uint16_t* q, const uint16_t* K, const uint16_t* V, const float* W,
                          uint32_t* codes, int B, int Hq, int Hkv, int64_t q_rows, int64_t cap,
                          const int32_t* seq_lens, int max_len, float scale, float* out, int r,
                          hipStream_t s, const PageMap* pm) {
  const int G = Hq / Hkv;
  PrefillArgs a;
  a.q = q; a.K = K; a.V = V; a.W = W; a.codes = codes; a.seq_lens = seq_lens; a.out = out;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.q_rows = q_rows; a.cap = cap; a.max_len = max_len;
  a.nqb = (max_len + 128 / G - 1) / (128 / G);
  a.scale_log2 = scale * 1.4426950408889634f;
  if (pm && pm->bt) {
    a.pm = *pm;
    return launch_p<true>(a, G, r, s);
  }
  a.pm = PageMap();
  return launch_p<false>(a, G, r, s);
}

}  // namespace hata
