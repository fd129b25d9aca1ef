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
// 8 the block -> unit map gives a unit only blocks whose indices agree mod 8;
// the dispatcher deals blocks round-robin over the 8 XCDs, so a unit's
// workgroups usually share one XCD and one L2.  Each workgroup stamps its XCD
// id into the workspace early in the launch and, before its first exchange,
// reads the stamps of its unit: when all of them show its own XCD, its
// exchange stores are plain stores (they land in that L2, where the readers'
// device-coherent loads find them); otherwise they are device-coherent.
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
// Exchanges between workgroups use stores into their own slots plus one
// monotonically increasing flag per workgroup; there is no same-address
// read-modify-write (those serialise at the memory side).  Every wait is
// bounded: a wait that gives up sets bit 0 of the workspace error word and
// the workgroup writes NaN into the unit's outputs and -2 into its kept
// indices instead of results built from incomplete data.
#include <atomic>
#include <mutex>

#include "hata_device.hpp"
#include "hata_launch.hpp"

// Scratch of hata_decode_step_noalloc: the decode step's workspace for
// callers that cannot allocate (zero at load; each device holds its own copy
// until the process ends).  Host code reaches it only through the address
// hipGetSymbolAddress returns for the current device (noalloc_scratch).
static __device__ __align__(256) unsigned char scratch[hata::kNoAllocScratchBytes];

namespace hata {

namespace {

constexpr int kMaxWg = 64;         // workgroups per unit (one polling wave)
constexpr int kWinBytes = 256;     // published window record per workgroup
constexpr int kWinWords = kWinBytes / 4;
constexpr int kWinHdr = 8;         // uint16 header entries
constexpr int kWinCap = kWinBytes / 2 - kWinHdr;  // histogram bins a window holds
constexpr int kMaxChunk = 32768;   // tokens per workgroup (uint16 scores in LDS)
constexpr int kStepWgMaxOcc2 = 32; // workgroups per unit when two share a CU
constexpr size_t kLdsPerCu = 160 * 1024;
constexpr uint32_t kSpinLimit = 1u << 22;  // default bound on the polls of one wait
// s_getreg operand for HW_REG_XCC_ID (register 20, bits 0..31): the XCD the
// wave runs on
constexpr int kXccIdReg = 20 | (31 << 11);
constexpr int kMaxPgl = kMaxChunk / 16 + 8;   // page ids of one chunk (pages of >= 16 rows)
constexpr int kPglPerThread = (kMaxPgl + kNT - 1) / kNT;

// Phase-trace build (compiled with HATA_PHASE_TRACE, a separate library used
// only for measurement): thread 0 of every workgroup reads the 100 MHz
// real-time counter at the phase boundaries listed below and stores the
// readings at exit.  Marks sit where the kernel already synchronises, so
// they add no barrier.
constexpr int kTracePoints = 24;
enum TracePoint {
  kTrStart = 0,      // first instruction
  kTrQcodes = 1,     // query codes built
  kTrScanned = 2,    // every owned token scored (appended key included)
  kTrHist = 3,       // cumulative histogram built
  kTrPublished = 4,  // window and flag stored
  kTrWait1 = 5,      // every window of the unit published
  kTrWindows = 6,    // windows read, headers parsed
  kTrThreshold = 7,  // threshold and this workgroup's tie quota known
  kTrCompacted = 8,  // kept list built
  kTrAttended = 9,   // attention over the kept rows done
  kTrRecord = 10,    // partial record and flag stored
  kTrWait2 = 11,     // every record of the unit published
  kTrEnd = 12,       // outputs written
  kTrQrows = 13,     // query rows staged in LDS
  kTrSearchLoop = 14,  // search bounds read, first round starts
  kTrRound1 = 15,    // first search round's partial counts exchanged in LDS
  kTrSearch = 16,    // threshold found (before the writers' prefix counts)
  kTrGathered = 17,  // first batch of kept K/V rows staged (G > 1)
  kTrAccum = 18      // every kept row accumulated, before the heads' merge (G > 1)
};
#ifdef HATA_PHASE_TRACE
#define HATA_MARK(i) \
  do {                                                        \
    if (threadIdx.x == 0) tr_ts[i] = __builtin_amdgcn_s_memrealtime(); \
  } while (0)
// a value recorded in slot i (slots 20..23: search rounds, window base,
// smallest own k-th score, threshold | kept rows << 16)
#define HATA_VALUE(i, v) \
  do {                                                        \
    if (threadIdx.x == 0) tr_ts[i] = (uint64_t)(v);           \
  } while (0)
#define HATA_TRACE_STORE()                                                     \
  do {                                                                         \
    if (threadIdx.x == 0) {                                                    \
      uint64_t* tr_dst = a.trace + ((int64_t)unit * a.Wg + w) * kTracePoints;  \
      for (int tr_i = 0; tr_i < kTracePoints; ++tr_i) tr_dst[tr_i] = tr_ts[tr_i]; \
    }                                                                          \
  } while (0)
#else
#define HATA_MARK(i) do {} while (0)
#define HATA_VALUE(i, v) do {} while (0)
#define HATA_TRACE_STORE() do {} while (0)
#endif

template <int G, int R = kR, bool PAGED = false>
struct Cfg {
  static constexpr int W64 = Width<R>::W64;       // 64-bit words per code row
  static constexpr int NB = G * R + 1;            // histogram bins
  static constexpr int NBP = (NB + 63) / 64 * 64;
  // code rows in flight per thread (8 rows of 8 or 16 bytes, 4 of 32: a
  // ring of 16 or 32 KiB per workgroup); deeper rings delay W_H, which
  // shares the CU's vector-memory path (16 rows of 8 bytes measured slower
  // at 128K than 8)
  static constexpr int PF = (R <= 128) ? 8 : 4;
  static constexpr int HDRP = (2 * G + 3) / 4 * 4; // partial record header floats (M[G], L[G])
  static constexpr int RECP = HDRP + G * kD;       // partial record floats
  static constexpr int PROJ = 4 * (G + 1) * R;     // projection reduction floats
  static constexpr int RED0 = (kMergeFloats<G> > PROJ) ? kMergeFloats<G> : PROJ;
  static constexpr int RED = (RED0 > (G + 4) * kRec) ? RED0 : (G + 4) * kRec;
  // LDS offsets in bytes
  // score histogram copies: one per wave (fewer same-address LDS atomics;
  // measured 0.2 us faster at 32K and 128K) when the bins are few, else one
  static constexpr int HCOPY = (NB <= 1024) ? 4 : 1;
  static constexpr int o_hist = 0;                               // HCOPY * NBP uint32
  static constexpr int NSTG = (G + 1 + 3) / 4;                   // staging loads per thread
  static constexpr int o_qf = o_hist + HCOPY * NBP * 4;          // 4*NSTG rows of 128 float (G+1 used)
  static constexpr int o_red = o_qf + 4 * NSTG * kD * 4;         // RED float
  static constexpr int o_qcode = (o_red + RED * 4 + 15) / 16 * 16;  // (G+1)*W64 uint64
  // (rounded up to 16 bytes: with one 64-bit word per code the query codes
  // end 8 bytes past a 16-byte boundary, and every later area is read with
  // 16-byte LDS accesses)
  static constexpr int o_misc = (o_qcode + (G + 1) * W64 * 8 + 15) / 16 * 16;  // 64 uint32
  static constexpr int o_whdr = o_misc + 64 * 4;                 // kMaxWg int4 + 2*4*64 uint32
  // the unit's histogram windows (read after the first exchange, used up by
  // the threshold) and the attention's staged K/V rows share one area, as
  // do the partial records staged for the final merge (after the attention)
  static constexpr int o_win = o_whdr + 4 * kMaxWg * 4 + 2048;   // kMaxWg*kWinBytes (also combine staging)
  static constexpr int o_kvs = o_win;                            // staged K rows and V^T of one batch
  static constexpr int WKV = (kMaxWg * kWinBytes > kMxLdsBytes) ? kMaxWg * kWinBytes : kMxLdsBytes;
  static constexpr int o_pgl = o_kvs + WKV;                      // paged: kMaxPgl int32 page ids
  static constexpr int o_sel = o_pgl + (PAGED ? kMaxPgl * 4 : 0); // k + 1 int32
  static_assert(o_qf % 16 == 0 && o_red % 16 == 0 && o_qcode % 16 == 0 && o_misc % 16 == 0 &&
                    o_whdr % 16 == 0 && o_win % 16 == 0 && o_pgl % 16 == 0 && o_sel % 16 == 0,
                "LDS areas start on 16-byte boundaries");
  static size_t lds_bytes(int k, int chunk) {
    size_t s = (size_t)o_sel + (size_t)(k + 1) * 4;
    s = (s + 15) / 16 * 16;
    // scores, padded to a multiple of 8 slabs of 256 tokens, with 8 spare
    // slots after every 128 tokens (sc_slot)
    return s + (size_t)((chunk + 8 * kNT - 1) / (8 * kNT) * (8 * kNT)) * 2 * 17 / 16;
  }
};

struct StepArgs {
  const uint16_t* q;
  const uint16_t* K;
  const uint16_t* V;
  const float* W;
  const float* Wk;  // key encoder (== W unless a separate one is given)
  uint32_t* codes;  // rows of W32 32-bit words
  const int32_t* seq_lens;
  float* out;
  int32_t* idx_out;
  int64_t cap;
  int Hq, Hkv, k;
  float scale;
  int Wg, chunk, xcd_map, U;
  // err[0]: error bits; err[1]: bound on the polls of one wait (0: the
  // default kSpinLimit); err[2]: never written in practice (see `warm`)
  uint32_t* err;
  uint32_t* stamps; // [U][kMaxWg]: (epoch << 4) | XCD id of each workgroup
#ifdef HATA_PHASE_TRACE
  uint64_t* trace;  // [U * Wg][kTracePoints] timestamps (phase-trace build only)
#endif
  uint32_t* flags;  // [U][kMaxWg]
  uint32_t* win;    // [U][kMaxWg][kWinWords]
  uint32_t* full;   // [U][kMaxWg][full_words]  (only for overflowing windows)
  float* part;      // [U][kMaxWg][RECP]
  int full_words;
  // paged cache (the PAGED instance): row j of (b, h) is row j % P of page
  // bt[b * max_pages + j / P] of pools [num_pages][Hkv][P][.], P = 2^log2P >= 16
  const int32_t* bt;
  int max_pages, num_pages, log2P;
};

// Block -> (unit, workgroup).  xcd_map: blocks agreeing mod 8 form the
// units of one XCD class (unit = 8 * (slot / Wg) + bid % 8, slot = bid / 8);
// otherwise unit = bid / Wg.  Branch-free, so the compiler issues every
// kernel-argument load at once (with a branch here it sank the load of the
// data pointers below the first argument wait).
__device__ __forceinline__ void map_block(const StepArgs& a, int* unit, int* w) {
  const int bid = blockIdx.x;
  const int sh = a.xcd_map ? 3 : 0;
  const int xcd = bid & ((1 << sh) - 1), slot = bid >> sh;
  const int uix = slot / a.Wg;
  *w = slot - uix * a.Wg;
  *unit = (uix << sh) + xcd;
}

// Wave 0 waits until every flag of the unit has reached `target`, for at
// most `limit` polls.  Returns true in every thread when it did; on a
// timeout bit 0 of the error word and *failed (LDS, preset to 0) are set.
__device__ __forceinline__ bool wait_unit(const StepArgs& a, int unit, uint32_t target, uint32_t limit,
                                          uint32_t* failed) {
  const int lane = threadIdx.x & 63;
  if ((threadIdx.x >> 6) == 0) {
    const CohBuf fb(a.flags + (int64_t)unit * kMaxWg, kMaxWg * 4);
    uint32_t it = 0;
    while (true) {
      const uint32_t v = (lane < a.Wg) ? fb.ld4(lane * 4) : target;
      const bool ok = (int32_t)(v - target) >= 0;
      if (__all(ok)) break;
      if (++it > limit) {
        if (lane == 0) {
          atomicOr(a.err, 1u);
          *failed = 1u;
        }
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __syncthreads();
  return *failed == 0u;
}

// In-place inclusive scan of hist[0, NB) with 256 threads (the sum of
// COPIES copies STRIDE words apart, written to the first).  Also records the
// first bin where the running count becomes > 0, >= cnt and >= k in misc[0],
// misc[1], misc[2] (each written by the one thread that sees the transition;
// the caller presets them to NB).  Ends with __syncthreads.
template <int NB, int COPIES = 1, int STRIDE = 0>
__device__ __forceinline__ void cum_hist(uint32_t* hist, uint32_t* misc, uint32_t* tmp,
                                         uint32_t cnt, uint32_t k) {
  constexpr int BPT = (NB + kNT - 1) / kNT;
  const int t = threadIdx.x;
  uint32_t v[BPT];
  uint32_t loc = 0;
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    const int s = t * BPT + j;
    uint32_t x = 0u;
    if (s < NB) {
#pragma unroll
      for (int c = 0; c < COPIES; ++c) x += hist[c * STRIDE + s];
    }
    v[j] = x;
    loc += v[j];
  }
  uint32_t tot;
  uint32_t prev = block_excl_scan_u32(loc, tmp, &tot);
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    const int s = t * BPT + j;
    if (s < NB) {
      const uint32_t run = prev + v[j];
      hist[s] = run;
      if (prev == 0 && run > 0) misc[0] = s;
      if (prev < cnt && run >= cnt) misc[1] = s;
      if (prev < k && run >= k) misc[2] = s;
      prev = run;
    }
  }
  __syncthreads();
}

// SEP: the appended key row is encoded with a separate key encoder a.Wk
// (a separate instance, so the shared-encoder code is unchanged).  R: code
// width in bits (32, 64, 128, 256).
// PAGED: K, V and codes are page pools addressed through a.bt (separate
// instance; the contiguous code is unchanged).
// Instances with G <= 4 and R <= 128 are compiled for two workgroups per CU
// (at most 256 registers a lane), which the plan uses for many units.
template <int G, int R>
constexpr int step_occupancy() { return (G <= 4 && R <= 128) ? 2 : 1; }

template <int G, bool SEP, int R, bool PAGED>
__global__ __launch_bounds__(kNT, (step_occupancy<G, R>())) void decode_step_kernel(const StepArgs a) {
  using C = Cfg<G, R, PAGED>;
  constexpr int W64 = C::W64, W32 = Width<R>::W32;
  constexpr int NB = C::NB;
  constexpr int PF = C::PF;
  extern __shared__ __align__(16) unsigned char smem[];
  uint32_t* hist = reinterpret_cast<uint32_t*>(smem + C::o_hist);
  float* qf = reinterpret_cast<float*>(smem + C::o_qf);
  float* red = reinterpret_cast<float*>(smem + C::o_red);
  uint64_t* qcode = reinterpret_cast<uint64_t*>(smem + C::o_qcode);
  uint32_t* misc = reinterpret_cast<uint32_t*>(smem + C::o_misc);
  int32_t* whdr = reinterpret_cast<int32_t*>(smem + C::o_whdr);  // writer headers + partial counts
  unsigned char* winb = smem + C::o_win;
  unsigned char* kvs = smem + C::o_kvs;
  int32_t* sel = reinterpret_cast<int32_t*>(smem + C::o_sel);
  uint16_t* sc = reinterpret_cast<uint16_t*>(smem + ((C::o_sel + (a.k + 1) * 4 + 15) / 16 * 16));
  // LDS slot of token li's score: 8 spare slots after every 128 tokens, so
  // that the compaction's 16-byte reads (thread t reading its run of
  // consecutive tokens from t * run on) fall on distinct bank groups for
  // runs of 32 tokens and more as well (unpadded, runs of 128 tokens put 8
  // consecutive lanes on one bank group); 8-token groups stay contiguous
  // and 16-byte aligned
  const auto sc_slot = [](int li) { return li + ((li >> 7) << 3); };

  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
#ifdef HATA_PHASE_TRACE
  uint64_t tr_ts[kTracePoints] = {};
#endif
  HATA_MARK(kTrStart);
  int unit, w;
  map_block(a, &unit, &w);
  const int b = unit / a.Hkv, h = unit - b * a.Hkv;
  const int64_t cap = a.cap;
  const int k = a.k;
  const int64_t row0 = PAGED ? 0 : ((int64_t)b * a.Hkv + h) * cap;
  // PAGED: physical row of logical row r of this unit, for a uniform r (one
  // scalar load of the page id; the page index is clamped into the table and
  // the id into the pool)
  auto prow = [&](int r) -> int64_t {
    const int pg = min(r >> a.log2P, a.max_pages - 1);
    // read as a constant (a scalar load, counted apart from the vector
    // loads, so using it does not wait for W_H and the code ring)
    typedef const __attribute__((address_space(4))) int32_t* cbt_p;
    const int pid = min(max(*(cbt_p)(a.bt + (int64_t)b * a.max_pages + pg), 0), a.num_pages - 1);
    return (((int64_t)pid * a.Hkv + h) << a.log2P) + (r & ((1 << a.log2P) - 1));
  };
  int32_t* pgl = reinterpret_cast<int32_t*>(smem + C::o_pgl);  // PAGED: the chunk's page ids
  // PAGED: page ids t, t + 256, ... of the chunk (0 past its pages), stored
  // into the LDS list with the staging
  int pgv[kPglPerThread] = {};
  // PAGED: page ids of the chunk's 256-row batches l and l + 64 in lane l of
  // every wave (a chunk has at most 128 batches), so a ring refill takes its
  // id with a readlane instead of a scalar load, whose wait would also drain
  // the scan's LDS atomics
  // The block-table words are loaded here, every load unconditional with its
  // index clamped into the table, and clamped into the pool only after the
  // query rows and W_H have been requested (below): a load whose value is
  // used at once, or under a branch, is followed by a wait for every load
  // before it, which with one wait per page id put eight round trips in
  // front of the code stream.
  int bpid0 = 0, bpid1 = 0;
  int npg = 0;
  if constexpr (PAGED) {
    const int32_t* btb = a.bt + (int64_t)b * a.max_pages;
    const int fp = (w * a.chunk) >> a.log2P;
    npg = ((w * a.chunk + a.chunk - 1) >> a.log2P) - fp + 1;
#pragma unroll
    for (int u = 0; u < kPglPerThread; ++u) pgv[u] = btb[min(fp + t + kNT * u, a.max_pages - 1)];
    // pages of >= 256 rows: the batch ids (otherwise never used)
    bpid0 = btb[min((w * a.chunk + lane * kNT) >> a.log2P, a.max_pages - 1)];
    bpid1 = btb[min((w * a.chunk + (lane + 64) * kNT) >> a.log2P, a.max_pages - 1)];
  }
  // PAGED: the ids of the chunk's pages lane and 64 + lane, in every wave
  // (the code ring's first PF batches of 256 rows lie in the first 128
  // pages for pages of >= 16 rows)
  int ppid0 = 0, ppid1 = 0;
  if constexpr (PAGED) {
    const int32_t* btb = a.bt + (int64_t)b * a.max_pages;
    const int fp = (w * a.chunk) >> a.log2P;
    ppid0 = btb[min(fp + lane, a.max_pages - 1)];
    ppid1 = btb[min(fp + 64 + lane, a.max_pages - 1)];
  }
  auto clamp_pid = [&](int v) { return min(max(v, 0), a.num_pages - 1); };
  // PAGED: physical row of the chunk's row lo + i for a uniform, 256-aligned
  // i < 32768 + BATCH (batch i / 256 of the chunk)
  auto prow_batch = [&](int lo_, int i) -> int64_t {
    const int bi = i >> 8;
    const int pid = __builtin_amdgcn_readlane(bi < 64 ? bpid0 : bpid1, bi & 63);
    return (((int64_t)pid * a.Hkv + h) << a.log2P) + ((lo_ + i) & ((1 << a.log2P) - 1));
  };
  // PAGED, pages of < 256 rows: physical row of this lane's row lo + i + t
  // from the chunk's page list in LDS (the index clamped into the list)
  auto prow_lane = [&](int lo_, int i) -> int64_t {
    const int r = lo_ + i + t;
    const int pi = min(max((r >> a.log2P) - (lo_ >> a.log2P), 0), kMaxPgl - 1);
    return (((int64_t)pgl[pi] * a.Hkv + h) << a.log2P) + (r & ((1 << a.log2P) - 1));
  };

  // ---- 1. loads.  The query rows, W_H, this workgroup's flag, the first
  // PF*256 rows of its code chunk and its exchange lines do not depend on
  // the sequence length, so they are issued before it is read; the appended
  // key row follows (only the workgroup that owns it waits for it, after its
  // scan).  Every load here is unconditional (clamped to a valid row, or to
  // a zero-size buffer that returns 0), so the compiler can count the loads
  // in flight exactly and wait for the early ones without draining the ring.
  // staging slot i of thread t holds dword (t + 256 i) % 64 of row (t + 256 i) / 64
  uint32_t xrow[C::NSTG];
#pragma unroll
  for (int i = 0; i < C::NSTG; ++i) {
    const int e = t + i * kNT;
    const int r = min(e >> 6, G - 1), c2 = e & 63;
    xrow[i] = 0;
    if (i * kNT < 64 * G)  // slots that hold query rows (known at compile time)
      xrow[i] = reinterpret_cast<const uint32_t*>(a.q + ((int64_t)b * a.Hq + (int64_t)h * G + r) * kD)[c2];
  }
  WRegs<R> wr;
  load_w_regs<R>(a.W + (int64_t)h * kD * R, wr);
  const uint32_t epoch =
      CohBuf(a.flags + (int64_t)unit * kMaxWg, a.Wg > 1 ? kMaxWg * 4 : 0).ld4(w * 4);
  // An invalid length is handled after the projection (below); until then
  // the length is clamped into [1, cap] so that every address is valid and
  // no branch stands between the loads above and their issue.
  const int lo = w * a.chunk;
  // the code ring's first PF*256 rows of the chunk, clamped into the cache
  // (rows past the sequence end are loaded and never scored)
  const uint32_t* cunit = a.codes + row0 * W32;
  CodeRow<R> cbuf[PF];
  if constexpr (PAGED) {
    // the page of row lo + j*256 + t, i.e. the chunk's page pi =
    // (row >> log2P) - (lo >> log2P) < 128, taken from lane pi % 64 of
    // ppid0 / ppid1 by a wave-local permute: one path for every page size,
    // with no branch and no load whose value is used at once, so the wait
    // for these ids (loaded ahead of the query rows and W_H) does not also
    // wait for those.  Rows past the cache are clamped to its last row
    // (loaded, never scored).
    bpid0 = clamp_pid(bpid0);
    bpid1 = clamp_pid(bpid1);
    const int fp = lo >> a.log2P;
#pragma unroll
    for (int j = 0; j < PF; ++j) {
      const int r = (int)min((int64_t)lo + j * kNT + t, cap - 1);
      const int pi = min(max((r >> a.log2P) - fp, 0), 127);
      const int v0 = __builtin_amdgcn_ds_bpermute((pi & 63) << 2, ppid0);
      const int v1 = __builtin_amdgcn_ds_bpermute((pi & 63) << 2, ppid1);
      const int pid = clamp_pid(pi < 64 ? v0 : v1);
      cbuf[j] = load_code<R>(a.codes, (((int64_t)pid * a.Hkv + h) << a.log2P) + (r & ((1 << a.log2P) - 1)));
    }
  } else {
#pragma unroll
    for (int j = 0; j < PF; ++j) cbuf[j] = load_code<R>(cunit, min((int64_t)lo + j * kNT + t, cap - 1));
  }
  // This workgroup's exchange lines (its histogram window and its partial
  // record) have usually left L2 since the previous step; the unit's first
  // reads of them after the flag take about 1 us then, against about 0.4 us
  // when the lines were loaded into L2 before this workgroup stores to them
  // (measured at 128K), so they are loaded here.  The values are consumed
  // only at the end of the kernel, so no wait is placed on these loads.
  uint32_t warm;
  {
    // one buffer over [win, end of the partial records); wave 0 touches the
    // window's 2 lines, the other waves the record's lines.  With one
    // workgroup per unit there is no exchange: a zero-size buffer.
    constexpr int plines = (C::RECP * 4 + 127) / 128 + 1;
    const bool ex = a.Wg > 1;
    const char* wbase = ex ? reinterpret_cast<const char*>(a.win) : reinterpret_cast<const char*>(a.err);
    const uint32_t part_off = ex ? (uint32_t)(reinterpret_cast<const char*>(a.part) - wbase) : 0u;
    const uint32_t span = ex ? part_off + (uint32_t)a.U * kMaxWg * C::RECP * 4 : 0u;
    const uint32_t woff = (uint32_t)(unit * kMaxWg + w) * kWinBytes + (t & 1) * 128;
    const uint32_t rec0 = (uint32_t)(unit * kMaxWg + w) * C::RECP * 4;
    const uint32_t poff = part_off + min(rec0 / 128 * 128 + (uint32_t)(t % plines) * 128,
                                         (uint32_t)(unit * kMaxWg + kMaxWg) * C::RECP * 4 - 4);
    warm = CohBuf(wbase, span).ld4(wv == 0 ? woff : poff);
  }
  // keep the loads above ahead of the length read in the issued code
  __builtin_amdgcn_sched_barrier(0);
  // The length and the wait bound are read as constants (scalar loads, which
  // do not queue behind the vector loads above; this kernel never writes
  // either word).
  typedef const __attribute__((address_space(4))) int32_t* cint_p;
  typedef const __attribute__((address_space(4))) uint32_t* cuint_p;
  const int n_in = *(cint_p)(a.seq_lens + b);
  // bound on the polls of one exchange wait (err[1] == 0: the default)
  const uint32_t spin_w = *(cuint_p)(a.err + 1);
  const uint32_t spin_limit = spin_w ? spin_w : kSpinLimit;
  const bool bad_len = n_in < 1 || (int64_t)n_in > cap;
  const int n = bad_len ? 1 : n_in;
  const int cnt = max(0, min(n, lo + a.chunk) - lo);
  const bool owns_new = (n - 1 >= lo) && (n - 1 < lo + cnt);
  const int new_li = n - 1 - lo;
  // row n-1 of K (row 0 when this workgroup does not own it): dword `lane`
  const int64_t krow_at = PAGED ? prow(owns_new ? n - 1 : 0) : row0 + (owns_new ? n - 1 : 0);
  const uint32_t krow = reinterpret_cast<const uint32_t*>(a.K + krow_at * kD)[lane];
  // ring refills: rows lo + li for li < cnt
  const uint32_t* cbase = cunit + (int64_t)(cnt > 0 ? lo : 0) * W32;

  // ---- 2. encode the query rows.  Every staging slot is stored (slots past
  // the G query rows are zero), so no load is consumed under a branch.
#pragma unroll
  for (int i = 0; i < C::NSTG; ++i) {
    const int e = t + i * kNT;
    const int r = e >> 6, c2 = e & 63;
    const uint32_t v = (r < G) ? xrow[i] : 0u;
    qf[r * kD + 2 * c2] = bf16_lo(v);
    qf[r * kD + 2 * c2 + 1] = bf16_hi(v);
  }
  for (int i = t; i < C::HCOPY * C::NBP; i += kNT) hist[i] = 0;
  if (t < 64) misc[t] = (t < 3) ? (uint32_t)NB : 0u;
  if constexpr (PAGED) {
#pragma unroll
    for (int u = 0; u < kPglPerThread; ++u)
      if (t + kNT * u < kMaxPgl) pgl[t + kNT * u] = (t + kNT * u < npg) ? clamp_pid(pgv[u]) : 0;
  }
  __syncthreads();
  HATA_MARK(kTrQrows);
  project_pack<G, R>(wr, qf, red, qcode, G);
  HATA_MARK(kTrQcodes);
  // this workgroup's XCD stamp for the launch ((epoch + 1) << 4 | XCD id;
  // epochs are even, so a stamp is never 0, the value of a fresh workspace)
  const uint32_t own_xcc = (uint32_t)__builtin_amdgcn_s_getreg(kXccIdReg) & 0xFu;
  const uint32_t own_stamp = ((epoch + 1u) << 4) | own_xcc;
  if (a.Wg > 1 && t == 0) CohBuf(a.stamps + (int64_t)unit * kMaxWg, kMaxWg * 4).st4(w * 4, own_stamp);
  if constexpr (SEP) {
    // Independent query and key encoders (HashAttention summary page,
    // "Approach"): the workgroup that owns the appended row reloads W's
    // registers, no longer needed for the queries, with the key encoder's
    // rows; the loads are in flight during its scan.
    if (owns_new) load_w_regs<R>(a.Wk + (int64_t)h * kD * R, wr);
  }
  if (bad_len) {
    // invalid length: every workgroup of the unit leaves here, before any
    // exchange, so the unit's flags stay consistent; workgroup 0 clears the
    // outputs
    if (w == 0) {
      for (int e = t; e < G * kD; e += kNT)
        a.out[((int64_t)b * a.Hq + (int64_t)h * G) * kD + e] = 0.f;
      if (a.idx_out)
        for (int j = t; j < k; j += kNT) a.idx_out[(int64_t)unit * k + j] = -1;
    }
    return;
  }
  uint32_t qw[G][W32];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int wd = 0; wd < W32; ++wd) qw[g][wd] = (uint32_t)(qcode[g * W64 + (wd >> 1)] >> ((wd & 1) * 32));
  QMasks<G, R> qm;
  build_qmasks<G, R>(qw, qm);

  // ---- 3. score the owned tokens.  Each ring slot is scored, then refilled
  // with the load PF*256 tokens ahead.  Row n-1 is scored from the cache
  // like the others and corrected afterwards by the thread that scored it.
  auto score_one = [&](const CodeRow<R>& c, int li) {
    uint32_t cw[W32];
    code_words<R>(c, cw);
    const uint32_t s = gqa_hamming_w<G, R>(cw, qm);
    sc[sc_slot(li)] = (uint16_t)s;
    atomicAdd(&hist[(C::HCOPY > 1 ? wv * C::NBP : 0) + s], 1u);
  };
  constexpr int BATCH = PF * kNT;
  int base = 0;
  // one full batch whose successor is full as well: score each ring slot and
  // refill it with the row BATCH tokens ahead
  auto scan_batch = [&](int b0) {
#pragma unroll
    for (int j = 0; j < PF; ++j) {
      const int li = b0 + j * kNT + t;
      score_one(cbuf[j], li);
      if constexpr (PAGED)
        cbuf[j] = load_code<R>(a.codes, a.log2P >= 8 ? prow_batch(lo, b0 + j * kNT + BATCH) + t
                                                     : prow_lane(lo, b0 + j * kNT + BATCH));
      else
        cbuf[j] = load_code<R>(cbase, li + BATCH);
    }
  };
  // The appended key row is encoded by the one workgroup that owns it (the
  // other workgroups never wait for it).  When the chunk spans at least two
  // ring batches it is projected right after the first batch, while the
  // refills of the second are in flight (its row was requested before
  // them), instead of adding one encode to that workgroup's path between
  // its scan and its window.
  auto encode_key = [&]() {
    if (t < 64) {
      qf[G * kD + 2 * lane] = bf16_lo(krow);
      qf[G * kD + 2 * lane + 1] = bf16_hi(krow);
    }
    __syncthreads();
    project_pack<1, R>(wr, qf + G * kD, red, qcode + G * W64, 1);
  };
  bool key_encoded = false;
  if (base + 2 * BATCH <= cnt) {  // this batch and the next are full
    scan_batch(base);
    base += BATCH;
    if (owns_new) {
      encode_key();
      key_encoded = true;
    }
  }
  for (; base + 2 * BATCH <= cnt; base += BATCH) scan_batch(base);
  if (base + BATCH <= cnt) {  // a full batch, the next one partial or empty
#pragma unroll
    for (int j = 0; j < PF; ++j) {
      const int li = base + j * kNT + t;
      score_one(cbuf[j], li);
      if constexpr (PAGED) {
        const int64_t rr = a.log2P >= 8 ? prow_batch(lo, base + j * kNT + BATCH) + t
                                        : prow_lane(lo, base + j * kNT + BATCH);
        if (li + BATCH < cnt) cbuf[j] = load_code<R>(a.codes, rr);
      } else {
        if (li + BATCH < cnt) cbuf[j] = load_code<R>(cbase, li + BATCH);
      }
    }
    base += BATCH;
  }
  if (base < cnt) {  // the last, partial batch
#pragma unroll
    for (int j = 0; j < PF; ++j) {
      const int li = base + j * kNT + t;
      if (li < cnt) score_one(cbuf[j], li);
    }
  }
  if (owns_new) {
    // the key's code goes to the cache and its score replaces the one
    // computed from the stale cache row
    if (!key_encoded) encode_key();
    if (t < W32) a.codes[(PAGED ? prow(n - 1) : row0 + n - 1) * W32 + t] = code_word32(qcode + G * W64, t);
    if (t == new_li % kNT) {
      uint32_t cw[W32];
#pragma unroll
      for (int wd = 0; wd < W32; ++wd) cw[wd] = (uint32_t)(qcode[G * W64 + (wd >> 1)] >> ((wd & 1) * 32));
      const uint32_t s_old = sc[sc_slot(new_li)];
      const uint32_t s_new = gqa_hamming_w<G, R>(cw, qm);
      atomicSub(&hist[s_old], 1u);
      atomicAdd(&hist[s_new], 1u);
      sc[sc_slot(new_li)] = (uint16_t)s_new;
    }
  }
  // the unit's XCD stamps (wave 0, lane = workgroup), read while the
  // histogram is scanned
  uint32_t unit_stamp = own_stamp;
  if (a.Wg > 1 && wv == 0)
    unit_stamp = CohBuf(a.stamps + (int64_t)unit * kMaxWg, kMaxWg * 4).ld4(min(lane, a.Wg - 1) * 4);
  __syncthreads();
  HATA_MARK(kTrScanned);

  // ---- 4. threshold
  cum_hist<NB, C::HCOPY, C::NBP>(hist, misc, misc + 8, (uint32_t)cnt, (uint32_t)k);
  HATA_MARK(kTrHist);
  const int lo_w = (int)misc[0];   // first nonempty bin (NB if none)
  const int hi_w = (int)misc[1];   // last nonempty bin
  const int tk = (int)misc[2];     // own k-th smallest score (NB if cnt < k)
  // A wait that gave up: the unit's results would rest on incomplete
  // exchange data, so this workgroup writes NaN into every output of the
  // unit and -2 into its kept indices (its error bit is already set).
  auto fail_unit = [&]() {
    float* o = a.out + ((int64_t)b * a.Hq + (int64_t)h * G) * kD;
    for (int e = t; e < G * kD; e += kNT) o[e] = __uint_as_float(0x7FC00000u);
    if (a.idx_out)
      for (int j = t; j < k; j += kNT) a.idx_out[(int64_t)unit * k + j] = -2;
  };
  int T;
  uint32_t lt_all, quota, sel_before = 0, take_self;
  if (a.Wg == 1) {
    T = (cnt >= k) ? tk : NB - 1;
    lt_all = T > 0 ? hist[T - 1] : 0u;
    quota = (uint32_t)k - lt_all;
    const uint32_t eq_self = hist[T] - lt_all;
    take_self = eq_self < quota ? eq_self : quota;
  } else {
    // Plain exchange stores only when every workgroup of the unit has
    // stamped this launch from this XCD (then every reader shares this L2);
    // the decision is kept in LDS for the partial records of step 7.
    bool xl = false;
    if (wv == 0) {
      xl = __all(unit_stamp == own_stamp) != 0;
      if (lane == 0) misc[25] = xl ? 1u : 0u;
    }
    const CohBuf wbuf(a.win + (int64_t)unit * kMaxWg * kWinWords, kMaxWg * kWinBytes);
    // publish the window [wlo, top] of this workgroup's histogram
    const bool has_k = cnt >= k;
    const int top = (cnt == 0) ? -1 : (has_k ? tk : hi_w);
    const int wlo = (cnt == 0) ? 0 : lo_w;
    const int len = top - wlo + 1;
    const bool ovf = len > kWinCap;
    if (t < kWinBytes / 16) {
      uint32_t e16[8];
      if (t == 0) {
        e16[0] = (uint32_t)wlo; e16[1] = (uint32_t)(top + 1);
        e16[2] = has_k ? 1u : 0u; e16[3] = ovf ? 1u : 0u;
        // cumulative count at the window's last stored bin
        e16[4] = (len > 0) ? hist[wlo + min(len, kWinCap) - 1] : 0u; e16[5] = 0;
        e16[6] = 0; e16[7] = 0;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int j = 8 * t + e - kWinHdr;
          const int s2 = wlo + j;
          // cumulative count (tokens with score <= s2); past the window's
          // end the count at its last bin
          e16[e] = (j < kWinCap && len > 0) ? hist[min(s2, top)] : 0u;
        }
      }
      u32x4 v;
      v.x = e16[0] | (e16[1] << 16); v.y = e16[2] | (e16[3] << 16);
      v.z = e16[4] | (e16[5] << 16); v.w = e16[6] | (e16[7] << 16);
      wbuf.st16x(w * kWinBytes + t * 16, v, xl);
    }
    if (ovf) {
      const CohBuf fbuf(a.full + ((int64_t)unit * kMaxWg + w) * a.full_words, a.full_words * 4);
      for (int i = t; i < a.full_words; i += kNT) {
        uint32_t two[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int s2 = 2 * i + e;
          two[e] = (s2 < NB) ? hist[s2] : (uint32_t)cnt;
        }
        fbuf.st4x(i * 4, two[0] | (two[1] << 16), xl);
      }
    }
    wait_all_mem();
    __syncthreads();
    if (t == 0) CohBuf(a.flags + (int64_t)unit * kMaxWg, kMaxWg * 4).st4x(w * 4, epoch + 1, xl);
    HATA_MARK(kTrPublished);
    if (!wait_unit(a, unit, epoch + 1, spin_limit, misc + 24)) {
      fail_unit();
      return;
    }
    HATA_MARK(kTrWait1);

    // read every window of the unit: Wg*16 chunks of 16 bytes, all in flight
    {
      const int nchunks = a.Wg * (kWinBytes / 16);
      u32x4 v[4];
      // wave 0 also loads writer `lane`'s header chunk into registers
      u32x4 hv = {0u, 0u, 0u, 0u};
      if (wv == 0) hv = wbuf.ld16(min(lane, a.Wg - 1) * kWinBytes);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = t + i * kNT;
        if (c < nchunks) v[i] = wbuf.ld16(c * 16);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = t + i * kNT;
        if (c < nchunks) *reinterpret_cast<u32x4*>(winb + c * 16) = v[i];
      }
      // Writer headers, parsed by wave 0 from registers (lane = writer):
      // first bin lw, window length ln, count at the window's end topc,
      // overflow flag; published in LDS with the barrier below.
      if (wv == 0) {
        int lw = NB, tw = NB - 1, ln = 0, topc = 0;
        bool hw = false, ow = false;
        if (lane < a.Wg) {
          lw = min((int)(hv.x & 0xFFFFu), NB);
          tw = min((int)(hv.x >> 16) - 1, NB - 1);
          hw = (hv.y & 0xFFFFu) != 0;
          ow = ((hv.y >> 16) & 1u) != 0;
          ln = max(0, min(tw - lw + 1, kWinCap));
          topc = ln > 0 ? (int)(hv.z & 0xFFFFu) : 0;
        }
        reinterpret_cast<int4*>(whdr)[lane] = make_int4(lw, ln, topc, ow ? 1 : 0);
        // T cannot exceed any workgroup's own k-th smallest score
        const int tmin = wave_min_i((lane < a.Wg && hw) ? tw : NB - 1);
        const int glo = min(wave_min_i(lw), tmin);
        const bool any_ow = __ballot(ow) != 0;
        if (lane == 0) { misc[16] = (uint32_t)glo; misc[17] = (uint32_t)tmin; misc[18] = any_ow ? 1u : 0u; }
      }
    }
    __syncthreads();
    HATA_MARK(kTrWindows);
    const int4* hdr4 = reinterpret_cast<const int4*>(whdr);            // [kMaxWg]
    uint32_t* cpart = reinterpret_cast<uint32_t*>(whdr + 4 * kMaxWg);  // [2][4][64]
    const bool any_ow = misc[18] != 0;
    // cumulative count of writer ww at bin s2 (0 below its window, the
    // window's last count past its end); an overflowing window is read from
    // the writer's full cumulative histogram instead
    auto win_count = [&](const int4 hd, int ww, int s2) -> uint32_t {
      const int j = s2 - hd.x;
      const uint16_t* ent = reinterpret_cast<const uint16_t*>(winb + ww * kWinBytes) + kWinHdr;
      const uint32_t v = ent[min(max(j, 0), kWinCap - 1)];
      // branch-free select keeps the entry reads of several writers in flight
      const uint32_t below = (uint32_t)(j >> 31);  // all ones when j < 0
      const uint32_t past = (uint32_t)((hd.y - 1 - j) >> 31);  // all ones when j >= ln
      return ((v & ~past) | ((uint32_t)hd.z & past)) & ~below;
    };
    auto cumw = [&](int ww, int s2) -> uint32_t {
      const int4 hd = hdr4[ww];
      if (any_ow && hd.w) {
        const CohBuf fbuf(a.full + ((int64_t)unit * kMaxWg + ww) * a.full_words, a.full_words * 4);
        const int sc2 = min(max(s2, 0), NB - 1);
        const uint32_t v = (fbuf.ld4((sc2 >> 1) * 4) >> ((sc2 & 1) * 16)) & 0xFFFFu;
        return s2 < hd.x ? 0u : v;
      }
      return win_count(hd, ww, s2);
    };
    // T = smallest s in [glo, tmin] with C(s) = sum of the writers' counts
    // >= k, else tmin.  Bins are tried 64 at a time (lane = bin), each wave
    // summing every 4th writer; every wave then forms the same totals.
    const int glo = (int)misc[16], tmin = (int)misc[17];
    int Tw = tmin;
    const int nper = (a.Wg + 3) / 4;
    HATA_VALUE(21, glo);
    HATA_VALUE(22, tmin);
    HATA_MARK(kTrSearchLoop);
    for (int c0 = glo, rnd = 0; c0 <= tmin; c0 += 64, ++rnd) {
      HATA_VALUE(20, rnd + 1);
      const int s2 = c0 + lane;
      // writers wv, wv+4, ... in groups of 8 (unused header slots count 0)
      uint32_t part = 0;
      if (!any_ow) {
        for (int i0 = 0; i0 < nper; i0 += 8) {
          int4 hd[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) hd[u] = hdr4[wv + 4 * (i0 + u)];
#pragma unroll
          for (int u = 0; u < 8; ++u) part += win_count(hd[u], wv + 4 * (i0 + u), s2);
        }
      } else {
        for (int i = 0; i < nper; ++i) part += cumw(wv + 4 * i, s2);
      }
      uint32_t* cp = cpart + (rnd & 1) * 256;
      cp[wv * 64 + lane] = part;
      __syncthreads();
      if (rnd == 0) HATA_MARK(kTrRound1);
      const uint32_t C = cp[lane] + cp[64 + lane] + cp[128 + lane] + cp[192 + lane];
      const uint64_t hit = __ballot(C >= (uint32_t)k && s2 <= tmin);
      if (hit) {
        Tw = c0 + (int)__builtin_ctzll(hit);
        break;
      }
    }
    HATA_MARK(kTrSearch);
    // Every wave (lane = writer) forms the writers' below-T and tie counts
    // and their prefixes itself and takes this workgroup's values by
    // readlane: no LDS round trip and no barrier.
    const uint32_t l1 = (lane < a.Wg && Tw > 0) ? cumw(lane, Tw - 1) : 0u;
    const uint32_t e1 = (lane < a.Wg) ? cumw(lane, Tw) - l1 : 0u;
    const uint32_t il = wave_incl_scan_u32(l1);
    const uint32_t ie = wave_incl_scan_u32(e1);
    T = Tw;
    lt_all = (uint32_t)__builtin_amdgcn_readlane((int)il, 63);
    quota = (uint32_t)k - lt_all;
    const uint32_t pre_lt = (uint32_t)__builtin_amdgcn_readlane((int)(il - l1), w);
    const uint32_t pre_eq = (uint32_t)__builtin_amdgcn_readlane((int)(ie - e1), w);
    const uint32_t eq_self = (uint32_t)__builtin_amdgcn_readlane((int)e1, w);
    const uint32_t left = quota > pre_eq ? quota - pre_eq : 0u;
    take_self = eq_self < left ? eq_self : left;
    sel_before = pre_lt + (pre_eq < quota ? pre_eq : quota);
  }
  HATA_MARK(kTrThreshold);

  // ---- 5. ordered compaction of the kept tokens (index order).  Thread t
  // owns the run of `run` consecutive tokens from t*run and records, per 32
  // of them, which are strict (score < T) and which tied (score == T) as bit
  // masks with token p of the word at bit 31-p.  A token's rank among the
  // workgroup's strict (resp. tied) tokens is the block prefix of the
  // per-thread counts plus the set bits above it; it is kept if strict, or
  // tied with tied-rank < take_self, at position
  // strict-rank + min(tied-rank, take_self).  Only set bits are visited.
  constexpr int kRunWords = kMaxChunk / kNT / 32;  // mask words per thread
  const int per8 = (cnt + 8 * kNT - 1) / (8 * kNT);  // 16-byte score reads per thread
  const int run = per8 * 8;
  const int i_begin = t * run;  // the padded score area covers 256 * run tokens
  const int nvalid = max(0, min(cnt - i_begin, run));
  // Masks of 8 tokens at once from packed 16-bit arithmetic (scores and T
  // are below 2^15): the sign bit of s - T (resp. s - T - 1) in each 16-bit
  // half says s < T (resp. s <= T); a byte permute with its sign-extension
  // selectors turns the 4 sign bits of two words into 4 bytes of 0x00 or
  // 0xFF, one bit of each byte is kept at its token's position (token q of
  // the 8 at bit 7 - q), and a multiply by 0x01010101 adds the 4 bytes of
  // two such words into the top byte: token q at bit 31 - q.
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  const u16x2 tv0 = {(unsigned short)T, (unsigned short)T};
  const u16x2 tv1 = {(unsigned short)(T + 1), (unsigned short)(T + 1)};
  auto byte_mask = [](const uint32_t (&d)[4]) {
    // selectors 8..11: 0xFF where bit 15 / 31 of the second operand, then
    // bit 15 / 31 of the first operand, is set
    const uint32_t a = __builtin_amdgcn_perm(d[1], d[0], 0x0B0A0908u);  // tokens 0..3
    const uint32_t b = __builtin_amdgcn_perm(d[3], d[2], 0x0B0A0908u);  // tokens 4..7
    const uint32_t x = (a & 0x10204080u) | (b & 0x01020408u);
    return (x * 0x01010101u) >> 24;
  };
  uint32_t mlt[kRunWords], meq[kRunWords];
#pragma unroll
  for (int wi = 0; wi < kRunWords; ++wi) {
    uint32_t ml = 0, mle = 0;
    if (wi * 4 < per8) {
      auto masks8 = [&](const uint4 v) {  // the 8 tokens of one 16-byte score read
        const uint32_t wds[4] = {v.x, v.y, v.z, v.w};
        uint32_t dl[4], de[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const u16x2 s2 = __builtin_bit_cast(u16x2, wds[q]);
          dl[q] = __builtin_bit_cast(uint32_t, (u16x2)(s2 - tv0));
          de[q] = __builtin_bit_cast(uint32_t, (u16x2)(s2 - tv1));
        }
        ml = (ml << 8) | byte_mask(dl);
        mle = (mle << 8) | byte_mask(de);
      };
      if (G == 1 && wi * 4 + 4 <= per8) {
        // One query head per KV head, a full word: its four reads are issued
        // together (runs of 32 tokens and more, i.e. chunks of 8192 tokens
        // and more, which occur with one workgroup per unit).  Measured on
        // this instance only; the others keep one read at a time.
        uint4 v4[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) v4[c] = *reinterpret_cast<const uint4*>(sc + sc_slot(i_begin + wi * 32 + c * 8));
#pragma unroll
        for (int c = 0; c < 4; ++c) masks8(v4[c]);
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if (wi * 4 + c < per8) {
            const uint4 v = *reinterpret_cast<const uint4*>(sc + sc_slot(i_begin + wi * 32 + c * 8));
            const uint32_t wds[4] = {v.x, v.y, v.z, v.w};
            uint32_t dl[4], de[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const u16x2 s2 = __builtin_bit_cast(u16x2, wds[q]);
              dl[q] = __builtin_bit_cast(uint32_t, (u16x2)(s2 - tv0));
              de[q] = __builtin_bit_cast(uint32_t, (u16x2)(s2 - tv1));
            }
            ml = (ml << 8) | byte_mask(dl);
            mle = (mle << 8) | byte_mask(de);
          }
        }
      }
      // left-align (token p at bit 31-p) and drop tokens past cnt
      const int ntok = min(32, run - wi * 32);
      const int nv = max(0, min(32, nvalid - wi * 32));
      const uint32_t keep = nv == 0 ? 0u : (~0u << (32 - nv));
      ml = (ml << (32 - ntok)) & keep;
      mle = (mle << (32 - ntok)) & keep;
    }
    mlt[wi] = ml;
    meq[wi] = mle & ~ml;
  }
  uint32_t own_pk = 0;
#pragma unroll
  for (int wi = 0; wi < kRunWords; ++wi)
    own_pk += (uint32_t)__popc(mlt[wi]) | ((uint32_t)__popc(meq[wi]) << 16);
  uint32_t tot_pk;  // packed halves never exceed kMaxChunk
  const uint32_t before_pk = block_excl_scan_u32(own_pk, misc + 8, &tot_pk);
  const uint32_t tot_lt = tot_pk & 0xFFFFu, tot_eq = tot_pk >> 16;
  {
    uint32_t ltb = before_pk & 0xFFFFu, eqb = before_pk >> 16;
#pragma unroll
    for (int wi = 0; wi < kRunWords; ++wi) {
      if (wi * 32 < run) {
        uint32_t m = mlt[wi] | meq[wi];
        while (m) {
          const int bpos = 31 - __clz(m);  // highest set bit: earliest token
          const uint32_t above = (bpos == 31) ? 0u : (~0u << (bpos + 1));
          const uint32_t rl = ltb + (uint32_t)__popc(mlt[wi] & above);
          const uint32_t re = eqb + (uint32_t)__popc(meq[wi] & above);
          const bool islt = (mlt[wi] >> bpos) & 1u;
          if (islt || re < take_self)
            sel[min(rl + min(re, take_self), (uint32_t)k)] = lo + i_begin + wi * 32 + (31 - bpos);
          m &= ~(1u << bpos);
        }
        ltb += (uint32_t)__popc(mlt[wi]);
        eqb += (uint32_t)__popc(meq[wi]);
      }
    }
  }
  const int m_self = min(k, (int)(tot_lt + min(tot_eq, take_self)));
  __syncthreads();
  HATA_MARK(kTrCompacted);

  // ---- 6. gather-fused attention over the kept rows (G > 1: batches of 64
  // rows staged in LDS, the next batch's loads in flight while a batch is
  // used, logits and weighted values on the matrix cores; G = 1: rows
  // gathered straight into registers, three steps of 64 rows in flight)
  if constexpr (PAGED) {
    const PagedRows map{pgl, (w * a.chunk) >> a.log2P, a.log2P, a.Hkv, h, kMaxPgl - 1};
    if constexpr (G == 1)
      attend_rows_g1<4, 3>(qf, sel, m_self, n, a.K, a.V, a.scale, red, map);
    else
      attend_heads_mx<G>(qf, sel, m_self, n, a.K, a.V, a.scale, red, reinterpret_cast<uint16_t*>(kvs), map);
  } else {
    if constexpr (G == 1)
      attend_rows_g1<4, 3>(qf, sel, m_self, n, a.K + row0 * kD, a.V + row0 * kD, a.scale, red);
    else
      attend_heads_mx<G>(qf, sel, m_self, n, a.K + row0 * kD, a.V + row0 * kD, a.scale, red,
                         reinterpret_cast<uint16_t*>(kvs), SameRows(), [&](int i) {
                           if (i == 0) HATA_MARK(kTrGathered); else HATA_MARK(kTrAccum);
                         });
  }

  HATA_MARK(kTrAttended);
  HATA_VALUE(23, (uint32_t)T | ((uint32_t)m_self << 16));
  // kept indices, written once the attention no longer needs the LDS list
  // (coalesced, and no barrier waits on these stores)
  auto write_idx = [&]() {
    if (!a.idx_out) return;
    int32_t* idx_unit = a.idx_out + (int64_t)unit * k;
    for (int j = t; j < m_self; j += kNT)
      if (sel_before + (uint32_t)j < (uint32_t)k) idx_unit[sel_before + j] = sel[j];
    if (w == 0)
      for (int j = min(k, n) + t; j < k; j += kNT) idx_unit[j] = -1;
  };
  float* outp = a.out + ((int64_t)b * a.Hq + (int64_t)h * G) * kD;
  if (a.Wg == 1) {
    write_idx();
    for (int e = t; e < G * kD; e += kNT) {
      const int g = e / kD, c = e % kD;
      const float* r = red + g * kRec;
      outp[e] = (r[1] > 0.f) ? r[2 + c] / r[1] : 0.f;
    }
    HATA_MARK(kTrEnd);
    HATA_TRACE_STORE();
    return;
  }

  // ---- 7. publish this workgroup's record, wait, merge a slice of the outputs
  const bool xl2 = misc[25] != 0u;  // plain stores (see step 4)
  const CohBuf pbuf(a.part + (int64_t)unit * kMaxWg * C::RECP, kMaxWg * C::RECP * 4);
  for (int c = t; c < C::RECP / 4; c += kNT) {
    float f[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = 4 * c + e;
      float v = 0.f;
      if (i < C::HDRP) {
        if (i < G) v = red[i * kRec];
        else if (i < 2 * G) v = red[(i - G) * kRec + 1];
      } else {
        const int j = i - C::HDRP, g = j / kD, cc = j % kD;
        v = red[g * kRec + 2 + cc];
      }
      f[e] = v;
    }
    u32x4 v4;
    v4.x = __float_as_uint(f[0]); v4.y = __float_as_uint(f[1]);
    v4.z = __float_as_uint(f[2]); v4.w = __float_as_uint(f[3]);
    pbuf.st16x((w * C::RECP + 4 * c) * 4, v4, xl2);
  }
  wait_all_mem();
  __syncthreads();
  if (t == 0) CohBuf(a.flags + (int64_t)unit * kMaxWg, kMaxWg * 4).st4x(w * 4, epoch + 2, xl2);
  HATA_MARK(kTrRecord);
  if (!wait_unit(a, unit, epoch + 2, spin_limit, misc + 24)) {
    fail_unit();
    return;
  }
  HATA_MARK(kTrWait2);

  // slice [e0, e1) of the G*128 outputs, a multiple of 4 wide
  const int per_wg = ((G * kD + a.Wg - 1) / a.Wg + 3) / 4 * 4;
  const int e0 = min(G * kD, w * per_wg), e1 = min(G * kD, e0 + per_wg);
  const int hch = C::HDRP / 4, sch = (e1 - e0) / 4, nch = hch + sch;
  {
    u32x4 v[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int f = t + i * kNT;
      if (f < a.Wg * nch) {
        const int ww = f / nch, c = f - ww * nch;
        const int off = (c < hch) ? 4 * c : C::HDRP + e0 + 4 * (c - hch);
        v[i] = pbuf.ld16((ww * C::RECP + off) * 4);
      }
    }
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int f = t + i * kNT;
      if (f < a.Wg * nch) *reinterpret_cast<u32x4*>(winb + f * 16) = v[i];
    }
  }
  __syncthreads();
  const float* stage = reinterpret_cast<const float*>(winb);
  // Output e0 + eo is formed by one row of 16 lanes; lane j takes writers
  // j, j+16, j+32, j+48.  The row finds its head's maximum M over the
  // writers, rescales each writer's L and accumulator by exp(M_w - M) and
  // adds them in a fixed order (per lane, then across the row).
  {
    const int sub16 = t & 15, nout = e1 - e0;
    for (int eo = t >> 4; eo < nout; eo += kNT / 16) {
      const int g = (e0 + eo) / kD;
      float mw[kMaxWg / 16];
      float Mloc = -INFINITY;
#pragma unroll
      for (int q = 0; q < kMaxWg / 16; ++q) {
        const int ww = sub16 + 16 * q;
        mw[q] = (ww < a.Wg) ? stage[ww * nch * 4 + g] : -INFINITY;
        Mloc = fmaxf(Mloc, mw[q]);
      }
      const float M = row16_max_f(Mloc);
      float Ls = 0.f, A = 0.f;
#pragma unroll
      for (int q = 0; q < kMaxWg / 16; ++q) {
        const int ww = sub16 + 16 * q;
        if (ww < a.Wg && mw[q] != -INFINITY) {
          const float f = __expf(mw[q] - M);
          Ls = fmaf(stage[ww * nch * 4 + G + g], f, Ls);
          A = fmaf(stage[ww * nch * 4 + C::HDRP + eo], f, A);
        }
      }
      Ls = sum16(Ls);
      A = sum16(A);
      if (sub16 == 0) outp[e0 + eo] = (Ls > 0.f) ? A / Ls : 0.f;
    }
  }
  if (warm == 0x9E3779B9u && k < 0) a.err[2] = warm;  // keeps the exchange-line loads
  // keep every flag slot of the unit equal for the next launch (which may
  // use a different number of workgroups per unit)
  if (w == 0 && t >= a.Wg && t < kMaxWg)
    st_agent(a.flags + (int64_t)unit * kMaxWg + t, epoch + 2);
  write_idx();
  HATA_MARK(kTrEnd);
  HATA_TRACE_STORE();
}

}  // namespace

template <int G>
static void cfg_sizes(int r, int k, int chunk, size_t* lds, size_t* recp) {
  switch (r) {
    case 32: *lds = Cfg<G, 32>::lds_bytes(k, chunk); *recp = Cfg<G, 32>::RECP; break;
    case 64: *lds = Cfg<G, 64>::lds_bytes(k, chunk); *recp = Cfg<G, 64>::RECP; break;
    case 256: *lds = Cfg<G, 256>::lds_bytes(k, chunk); *recp = Cfg<G, 256>::RECP; break;
    default: *lds = Cfg<G, 128>::lds_bytes(k, chunk); *recp = Cfg<G, 128>::RECP; break;
  }
}

StepPlan plan_decode_step(int B, int Hq, int Hkv, int64_t max_len, int k, int num_cus, int r) {
  StepPlan p;
  p.R = r;
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
  // Two workgroups per CU (instances with G <= 4 and r <= 128 are built for
  // it) when a unit already spans several workgroups, that gives it at most
  // 32 and the LDS fits: smaller chunks, and one workgroup's waits overlap
  // the other's work (measured at 64K tokens, batch 4: 23.8 -> 20.2 us per
  // step).  Not beyond 32 workgroups per unit (at 64 the exchanges cost more
  // than that gains) and not from one (that adds both exchanges: MHA batch
  // 8, 40.7 -> 44.8 us).
  if (p.fused && p.G <= 4 && r <= 128 && Wg > 1) {
    int Wg2 = 2 * num_cus / (U > 0 ? U : 1);
    if (Wg2 > kStepWgMaxOcc2) Wg2 = kStepWgMaxOcc2;
    if (Wg2 > by_tokens) Wg2 = (int)by_tokens;
    int64_t chunk2 = (max_len + Wg2 - 1) / Wg2;
    chunk2 = (chunk2 + kNT - 1) / kNT * kNT;
    if (Wg2 > Wg && chunk2 <= kMaxChunk && (int64_t)U * Wg2 <= 2 * num_cus) {
      size_t l2 = 0, r2 = 0;
      switch (p.G) {
        case 1: cfg_sizes<1>(r, k, (int)chunk2, &l2, &r2); break;
        case 2: cfg_sizes<2>(r, k, (int)chunk2, &l2, &r2); break;
        default: cfg_sizes<4>(r, k, (int)chunk2, &l2, &r2); break;
      }
      if (l2 <= kLdsPerCu / 2) {
        Wg = Wg2;
        chunk = chunk2;
      }
    }
  }
  p.Wg = Wg;
  p.chunk = (int)chunk;
  p.xcd_map = (Wg > 1 && U % 8 == 0) ? 1 : 0;
  auto align = [](size_t x) { return (x + 255) / 256 * 256; };
  const int G = p.G;
  const int NB = G * r + 1;
  p.full_words = (NB + 1) / 2;
  size_t recp = 0;
  if (p.fused) {
    switch (G) {
      case 1: cfg_sizes<1>(r, k, p.chunk, &p.lds_bytes, &recp); break;
      case 2: cfg_sizes<2>(r, k, p.chunk, &p.lds_bytes, &recp); break;
      case 4: cfg_sizes<4>(r, k, p.chunk, &p.lds_bytes, &recp); break;
      default: cfg_sizes<8>(r, k, p.chunk, &p.lds_bytes, &recp); break;
    }
    // 160 KiB of LDS per CU, less the kernel's static LDS and a margin
    if (p.lds_bytes > 159 * 1024) p.fused = false;
  }
  size_t off = 0;
  p.off_err = off;   off = align(off + 256);
  // The exchange area (flags, stamps and histogram windows of every unit's
  // kMaxWg workgroup slots) sits at offsets that depend on the unit count
  // only and is reserved whether or not this call runs the fused step, so a
  // call that runs the separate kernels never writes over the flags that a
  // later fused step with the same B and Hkv reads its epoch from.
  const size_t slots = (size_t)U * kMaxWg;
  p.off_flags = off;  off = align(off + slots * 4);
  p.off_stamps = off; off = align(off + slots * 4);
  p.off_win = off;    off = align(off + slots * kWinWords * 4);
  p.off_xend = off;
  if (p.fused) {
    if (Wg > 1) {
      p.off_full = off; off = align(off + slots * (size_t)p.full_words * 4);
      p.off_part = off; off = align(off + slots * recp * 4);
    }
  } else {
    // staged steps inside hata_decode_step
    p.off_qc = off;     off = align(off + (size_t)B * Hq * ((r + 31) / 32) * 4);
    p.off_scores = off; off = align(off + (size_t)U * max_len * 2);
    p.off_idx = off;    off = align(off + (size_t)U * k * 4);  // kept list when idx_out is NULL
    p.off_attn = off;   off = align(off + attn_part_floats(B, Hkv, G, k) * 4);
    p.off_topk = off;   off = align(off + topk_scratch_bytes(B, Hkv, max_len, G * r));
  }
#ifdef HATA_PHASE_TRACE
  if (p.fused) {
    p.off_trace = off;
    off = align(off + (size_t)U * Wg * kTracePoints * 8);
  }
#endif
  p.total = off;
  return p;
}

template <int G, bool SEP, int R, bool PAGED = false>
static hipError_t launch_step_gsr(const StepPlan& p, const StepArgs& a, hipStream_t s) {
  const size_t lds = p.lds_bytes + (PAGED ? kMaxPgl * 4 : 0);
  // raise the kernel's dynamic-LDS limit when a plan needs more than 64 KiB
  static std::atomic<size_t> configured{64 * 1024};
  if (lds > configured.load()) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_step_kernel<G, SEP, R, PAGED>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    configured.store(lds);
  }
  hipLaunchKernelGGL((decode_step_kernel<G, SEP, R, PAGED>), dim3(p.U * p.Wg), dim3(kNT), lds, s, a);
  return hipGetLastError();
}

template <int G, bool SEP>
static hipError_t launch_step_gs(const StepPlan& p, const StepArgs& a, hipStream_t s) {
  switch (p.R) {
    case 32: return launch_step_gsr<G, SEP, 32>(p, a, s);
    case 64: return launch_step_gsr<G, SEP, 64>(p, a, s);
    case 256: return launch_step_gsr<G, SEP, 256>(p, a, s);
    default: return launch_step_gsr<G, SEP, 128>(p, a, s);
  }
}

template <int G>
static hipError_t launch_step_g(const StepPlan& p, const StepArgs& a, hipStream_t s) {
  return a.Wk == a.W ? launch_step_gs<G, false>(p, a, s) : launch_step_gs<G, true>(p, a, s);
}

hipError_t launch_decode_step(const StepPlan& p, const uint16_t* q, const uint16_t* K,
                              const uint16_t* V, const float* W, const float* Wk, uint32_t* codes, int B, int Hq,
                              int Hkv, int64_t cap, const int32_t* seq_lens, int k, float scale,
                              float* out, int32_t* idx_out, unsigned char* ws, hipStream_t s) {
  StepArgs a;
  a.q = q; a.K = K; a.V = V; a.W = W; a.Wk = Wk ? Wk : W; a.codes = codes; a.seq_lens = seq_lens;
  a.out = out; a.idx_out = idx_out; a.cap = cap; a.Hq = Hq; a.Hkv = Hkv; a.k = k;
  a.scale = scale; a.Wg = p.Wg; a.chunk = p.chunk; a.xcd_map = p.xcd_map; a.U = p.U;
  a.err = reinterpret_cast<uint32_t*>(ws + p.off_err);
  a.stamps = reinterpret_cast<uint32_t*>(ws + p.off_stamps);
#ifdef HATA_PHASE_TRACE
  a.trace = reinterpret_cast<uint64_t*>(ws + p.off_trace);
#endif
  a.flags = reinterpret_cast<uint32_t*>(ws + p.off_flags);
  a.win = p.Wg > 1 ? reinterpret_cast<uint32_t*>(ws + p.off_win) : nullptr;
  a.full = p.Wg > 1 ? reinterpret_cast<uint32_t*>(ws + p.off_full) : nullptr;
  a.part = p.Wg > 1 ? reinterpret_cast<float*>(ws + p.off_part) : nullptr;
  a.full_words = p.full_words;
  a.bt = nullptr; a.max_pages = 0; a.num_pages = 0; a.log2P = 0;
  (void)B;
  switch (p.G) {
    case 1: return launch_step_g<1>(p, a, s);
    case 2: return launch_step_g<2>(p, a, s);
    case 4: return launch_step_g<4>(p, a, s);
    case 8: return launch_step_g<8>(p, a, s);
    default: return hipErrorInvalidValue;
  }
}

template <int G>
static hipError_t launch_paged_g(const StepPlan& p, const StepArgs& a, hipStream_t s) {
  switch (p.R) {
    case 32: return launch_step_gsr<G, false, 32, true>(p, a, s);
    case 64: return launch_step_gsr<G, false, 64, true>(p, a, s);
    case 256: return launch_step_gsr<G, false, 256, true>(p, a, s);
    default: return launch_step_gsr<G, false, 128, true>(p, a, s);
  }
}

bool decode_step_paged_fusable(const StepPlan& p, int page_rows) {
  return p.fused && page_rows >= 16 && p.lds_bytes + kMaxPgl * 4 <= 159 * 1024;
}

hipError_t launch_decode_step_paged(const StepPlan& p, const uint16_t* q, const uint16_t* K, const uint16_t* V,
                                    const float* W, uint32_t* codes, const PageMap& pm, int Hq, int Hkv,
                                    const int32_t* seq_lens, int k, float scale, float* out, int32_t* idx_out,
                                    unsigned char* ws, hipStream_t s) {
  if (!decode_step_paged_fusable(p, 1 << pm.log2P)) return hipErrorInvalidValue;
  StepArgs a;
  a.q = q; a.K = K; a.V = V; a.W = W; a.Wk = W; a.codes = codes; a.seq_lens = seq_lens;
  a.out = out; a.idx_out = idx_out; a.cap = (int64_t)pm.max_pages << pm.log2P; a.Hq = Hq; a.Hkv = Hkv; a.k = k;
  a.scale = scale; a.Wg = p.Wg; a.chunk = p.chunk; a.xcd_map = p.xcd_map; a.U = p.U;
  a.err = reinterpret_cast<uint32_t*>(ws + p.off_err);
  a.stamps = reinterpret_cast<uint32_t*>(ws + p.off_stamps);
#ifdef HATA_PHASE_TRACE
  a.trace = reinterpret_cast<uint64_t*>(ws + p.off_trace);
#endif
  a.flags = reinterpret_cast<uint32_t*>(ws + p.off_flags);
  a.win = p.Wg > 1 ? reinterpret_cast<uint32_t*>(ws + p.off_win) : nullptr;
  a.full = p.Wg > 1 ? reinterpret_cast<uint32_t*>(ws + p.off_full) : nullptr;
  a.part = p.Wg > 1 ? reinterpret_cast<float*>(ws + p.off_part) : nullptr;
  a.full_words = p.full_words;
  a.bt = pm.bt; a.max_pages = pm.max_pages; a.num_pages = pm.num_pages; a.log2P = pm.log2P;
  switch (p.G) {
    case 1: return launch_paged_g<1>(p, a, s);
    case 2: return launch_paged_g<2>(p, a, s);
    case 4: return launch_paged_g<4>(p, a, s);
    case 8: return launch_paged_g<8>(p, a, s);
    default: return hipErrorInvalidValue;
  }
}

// Device address of `scratch` on the current device, looked up once per
// device (hipGetSymbolAddress with that device current) and kept.
hipError_t noalloc_scratch(unsigned char** out) {
  constexpr int kDevs = 64;
  static std::mutex mu;
  static unsigned char* ptrs[kDevs] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kDevs) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    ptrs[dev] = static_cast<unsigned char*>(p);
  }
  *out = ptrs[dev];
  return hipSuccess;
}

}  // namespace hata
