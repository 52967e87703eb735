// Lightning-indexer scoring on MFMA for decode-shaped work (row a2):
// I[t, s] = sum_h w[t, h] * ReLU(q[t, h] . K[s]) ("2026 DeepSeek-V4" note,
// "Key design 1" indexer equation; "DeepSeek-V4" book ch. 6 "The index
// score"), for d_I = 128 and H_I a multiple of 16 (<= 64).
//
// The scan over the visible keys is the HBM stream of a CSA decode step.  A
// wavefront owns a contiguous run of 16-key tiles and streams them in
// batches of kU tiles: every load instruction reads 1 KB of consecutive rows
// (full cache lines) into registers, and the next batch is in flight while
// the current one is scored, so a wavefront keeps up to 2 kU tiles of reads
// outstanding (registers hold far more in-flight data per CU than LDS
// could).  A batch is transposed to the MFMA operand layout through a
// per-wavefront LDS buffer (private to the wavefront, so only its own LDS
// counter is waited on); the 16-byte chunks of each key are stored XOR
// swizzled so that both the writes and the MFMA-layout reads hit distinct
// LDS banks.
//
// Scoring: C[heads x keys] = Q[heads x d] . K^T[d x keys] with Q in
// registers (v_mfma_f32_16x16x32_bf16, 4 k-steps, for bf16 keys; the scaled
// f8f6f4 v_mfma 16x16x128 with unit scales for e4m3 keys, one step, with the
// reduction index permuted so a lane takes bytes 16g.. and 64+16g.. of its
// key; the query operand uses the same permutation).  The accumulator holds 4
// heads x 1 key per lane, so ReLU, the head weights and the head sum are
// in-lane, then two cross-lane adds.  For e4m3 the per-head query scale is
// folded into w and the per-key scale multiplies the sum (both positive, so
// they commute with ReLU).  With use_hist the wave also counts the top 11
// bits of each score's order-preserving key into an LDS histogram that is
// added to the row's global histogram at the end (stage 1 of the top-k).
//
// Fused top-k collection (fuse, decode): every workgroup also keeps its
// scores in LDS.  When its histogram is added, it arrives on its row's
// counter; the last workgroup of the row reads the complete histogram,
// finds the threshold bin and publishes it; the others wait for that (the
// grid is one round of resident workgroups, so all of them are running; the
// wait is bounded and a row that times out falls back to a scan of its
// scores).  Each workgroup then writes its certain winners and threshold-bin
// candidates, in entry order, to its own region of the row's lists, with the
// counts in wg_info, and one workgroup per row merges the lists
// (topk_fused_resolve_kernel).  The scores are not read back from memory and
// no list reservation contends on a counter.
//
// Fold workgroup (fold_mode, decode with the fused collection): the last
// workgroup of each row scans nothing; it performs the step's compressor
// work for its sequence instead of a separate kernel: when the block ending
// at the query position completes, it folds the new indexer key (and
// stores it, e4m3-quantized or bf16), scores it against the query exactly
// as the scan would, and takes part in the histogram and the lists with that
// one entry (the highest id, so its list comes last); it folds the new main
// entry, appends the token to the tail rings and the window ring, and the
// last workgroup of the row to arrive publishes the new entry count (every
// workgroup of the row has read the old count by then).  The scan
// workgroups cover the entries before the new one.

#include <atomic>
#include <type_traits>

#include "common.h"
#include "fold.h"
#include "topk.h"

namespace csa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// ReLU as one integer max on the bit pattern: non-negative floats order
// like their bits, negative ones (sign bit set) are negative integers
CSA_DEV float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

namespace {

constexpr int kD = 128;
// the fold workgroup stages every source of a block at once when the block
// has at most kFastFoldM tokens per branch and kFastFoldC coordinates
constexpr int kFastFoldM = 4;
constexpr int kFastFoldC = 512;

// Key formats of the scan (FMT): 0 bf16, 1 e4m3 with a float32 scale per
// key, 2 MXFP4 (E2M1 pairs, one E8M0 scale per 32 values).
//
// Tile geometry.  e4m3: 16 keys x 128 B = 2 KB, read as two 1 KB pieces of
// 8 keys; bf16: 16 keys x 256 B = 4 KB, four pieces of 4 keys.  In LDS, chunk
// q of key (piece j, key-in-piece k) sits at chunk position kCpk*k + (q ^ s)
// of piece j, s = k ^ j (e4m3) or k + 4j (bf16).  MXFP4: 16 keys x 64 B =
// 1 KB, loaded straight into the MFMA operand layout (no LDS).
template <int FMT>
struct Geo {
  static constexpr int kKeyB = FMT == 2 ? 64 : (FMT == 1 ? 128 : 256);
  static constexpr int kTileB = 16 * kKeyB;
  static constexpr int kPieces = kTileB / 1024;
  static constexpr int kKpp = 16 / kPieces;  // keys per piece
  static constexpr int kCpk = kKeyB / 16;    // 16-byte chunks per key
  // tiles per batch (even).  bf16: two, so that the transpose buffers
  // (8 KB per wavefront) let two workgroups share a CU (measured on the
  // Flash CSA 128K step: 28.4 us against 29.8 us with four tiles and one
  // workgroup per CU)
  static constexpr int kU = FMT == 2 ? 8 : (FMT == 1 ? 6 : 2);
  // per-wavefront LDS: a batch's transpose buffer; MXFP4 needs none, only
  // room for the fold workgroup's staging (a quarter each)
  static constexpr int kTrB = FMT == 2 ? 8192 : kU * kTileB;
  CSA_DEV static int sw(int k, int j) { return FMT == 1 ? (k ^ j) : (k + 4 * j); }
  // LDS byte offset of chunk q of key c within a tile
  CSA_DEV static int lds_off(int c, int q) {
    const int j = c / kKpp, k = c % kKpp;
    return 1024 * j + 16 * (kCpk * k + (q ^ sw(k, j)));
  }
};

}  // namespace

// grid (n_wg, rows), 256 threads
// wait_polls: how many times a waiting workgroup polls for its row's
// published threshold bin before it gives up (a multiple of 4)
template <int FMT, int HT, int PG>
__global__ __launch_bounds__(256) void index_score_mfma_kernel(IndexArgs a, TopkWs ws, int use_hist, int fuse,
                                                                FoldArgs f, int fold_mode, int wait_polls) {
  constexpr bool FP8 = FMT == 1, FP4 = FMT == 2;
  typedef Geo<FMT> G;
  constexpr int kU = G::kU;
  __shared__ __attribute__((aligned(1024))) char s_tr[4][G::kTrB];  // per-wave transpose buffer
  __shared__ int s_hist[kTopkBins];
  __shared__ __attribute__((aligned(16))) float s_sc[kTopkFuseCap];  // fused: this workgroup's scores, by entry - first entry
  __shared__ int s_misc[16];
  const int row = blockIdx.y, b = row / a.Tq, tq = row % a.Tq;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, li = l & 15, lg = l >> 4;
  const int H = a.H_I;

  // query operands and head weights first: small, their loads go out
  // before the key stream so they do not queue behind it (the fold
  // workgroup does not scan and skips them)
  const bool is_fold_wg = fold_mode && blockIdx.x == gridDim.x - 1;
  bf16x8_t qb[HT][4];
  i32x8_t q8[HT];
  int qsc[HT];  // MXFP4: the E8M0 scale of the lane's query block
  float wr[HT][4];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    if (is_fold_wg) {
      q8[ht] = i32x8_t{0, 0, 0, 0, 0, 0, 0, 0};
      qsc[ht] = 127;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) qb[ht][ks] = bf16x8_t{};
      wr[ht][0] = wr[ht][1] = wr[ht][2] = wr[ht][3] = 0.f;
      continue;
    }
    const int h = 16 * ht + li;
    if constexpr (FP4) {
      // the lane's operand: block lg (32 values, 16 bytes) of head h, with
      // the block's scale
      const uint8_t* q = reinterpret_cast<const uint8_t*>(a.q) + ((size_t)row * H + h) * (kD / 2) + 16 * lg;
      const uint4 v = *reinterpret_cast<const uint4*>(q);
      q8[ht] = i32x8_t{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
      qsc[ht] = reinterpret_cast<const uint8_t*>(a.q_scale)[((size_t)row * H + h) * (kD / 32) + lg];
    } else if constexpr (FP8) {
      const uint8_t* q = reinterpret_cast<const uint8_t*>(a.q) + ((size_t)row * H + h) * kD + 16 * lg;
      const uint4 v0 = *reinterpret_cast<const uint4*>(q), v1 = *reinterpret_cast<const uint4*>(q + 64);
      q8[ht] = i32x8_t{(int)v0.x, (int)v0.y, (int)v0.z, (int)v0.w, (int)v1.x, (int)v1.y, (int)v1.z, (int)v1.w};
    } else {
      const uint16_t* q = reinterpret_cast<const uint16_t*>(a.q) + ((size_t)row * H + h) * kD;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) qb[ht][ks] = *reinterpret_cast<const bf16x8_t*>(q + 32 * ks + 8 * lg);
    }
    // heads 16 ht + 4 lg + r: one 16-byte load
    const float4 wv = *reinterpret_cast<const float4*>(a.w + (size_t)row * H + 16 * ht + 4 * lg);
    wr[ht][0] = wv.x; wr[ht][1] = wv.y; wr[ht][2] = wv.z; wr[ht][3] = wv.w;
  }
  // e4m3 always comes with its per-head query scale (bf16 never has one)
  float4 qs[HT];
  if constexpr (FP8) {
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
      qs[ht] = is_fold_wg ? make_float4(0.f, 0.f, 0.f, 0.f)
                          : *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(a.q_scale) +
                                                             (size_t)row * H + 16 * ht + 4 * lg);
  }
  __builtin_amdgcn_sched_barrier(0);

  // the visible-entry count (scalar loads), then the first two key batches
  const int64_t t = a.q_pos ? a.q_pos[(size_t)b * a.Tq + tq] : a.q_pos0 + tq;
  const int32_t n_have = a.n_entries[b];
  const int64_t lim = vis_limit(t, a.m, a.vis);
  // fold_mode: the block ending at t completes entry n_have in this step
  const bool fold_now = fold_mode && lim == (int64_t)n_have + 1 && n_have < a.E_cap;
  const bool fold_wg = is_fold_wg;
  int64_t nv = lim;  // visible entries, including a new one
  {
    const int64_t have = (int64_t)n_have + a.n_add + (fold_now ? 1 : 0);
    if (have < nv) nv = have;
    if (nv > a.E_cap) nv = a.E_cap;
    if (nv < 0) nv = 0;
  }
  const int64_t nv_scan = fold_now ? nv - 1 : nv;  // the scan workgroups' entries
  // PG (paged key cache): the pool's base; rows below come from the pages
  const size_t seq0 = PG ? 0 : (size_t)b * a.E_cap;
  const char* keys = reinterpret_cast<const char*>(a.keys) + seq0 * G::kKeyB;
  const float* ksc = FP8 ? reinterpret_cast<const float*>(a.k_scale) + seq0 : nullptr;
  const uint8_t* ksc4 = FP4 ? reinterpret_cast<const uint8_t*>(a.k_scale) + seq0 * (kD / 32) : nullptr;
  float* out = a.scores + (size_t)row * a.E_cap;

  // this wave's tiles [t0, t1), in batches of kU
  const int64_t ntile = (nv_scan + 15) / 16;
  const int64_t nwaves = (int64_t)(gridDim.x - fold_mode) * 4;
  const int64_t per = (ntile + nwaves - 1) / nwaves;
  const int64_t t0 = ((int64_t)blockIdx.x * 4 + w) * per;
  const int64_t t1 = t0 + per < ntile ? t0 + per : ntile;
  const int n = (t1 > t0 && !fold_wg) ? (int)(t1 - t0) : 0;
  const int nbatch = (n + kU - 1) / kU;

  // piece j of a tile: lane l reads bytes [16 l, 16 l + 16) of the piece,
  // i.e. chunk (l % kCpk) of key kKpp*j + l / kCpk; MXFP4: lane (li, lg)
  // reads block lg of key li, its MFMA operand (and that block's scale)
  typedef u32x4_t KBatch[kU][G::kPieces];
  typedef typename std::conditional<FP4, uint32_t, float>::type SBatch[kU];
  const int ld_key = FP4 ? li : l / G::kCpk, ld_chunk = FP4 ? lg : l % G::kCpk;
  // the last row of this wave's run: loads past it (the tail of the run and
  // the batches after it) all re-read that row, which stays in cache
  const int64_t e_last = (t1 * 16 < nv_scan ? t1 * 16 : nv_scan) - 1;
  // PG: lane i holds the page id of the run's page p_first + i (a run
  // spans at most 64 pages of >= 16 entries, which the launch checks); a
  // tile's 16 entries (and the clamped re-reads) share one page, whose id
  // a lane read takes from that register
  const int sh = a.pg.shift;
  const int64_t p_first = (t0 * 16) >> sh;
  int lane_pg = 0;
  if constexpr (PG) {
    if (n > 0) {
      const int64_t np_row = (int64_t)(a.E_cap >> sh);
      const int64_t p = p_first + l < np_row ? p_first + l : np_row - 1;
      lane_pg = a.pg.table[(size_t)b * np_row + p];
    }
  }
  auto load_batch = [&](KBatch& kreg, SBatch& sreg, int bi) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t e0 = (t0 + (int64_t)bi * kU + u) * 16;
      int64_t delta = 0;  // cache row - entry index for the tile's page
      if constexpr (PG) {
        const int64_t ee = e0 < e_last ? e0 : e_last;
        const int pid = __builtin_amdgcn_readlane(lane_pg, (int)((ee >> sh) - p_first));
        delta = ((int64_t)(uint32_t)pid - (ee >> sh)) << sh;
      }
#pragma unroll
      for (int j = 0; j < G::kPieces; ++j) {
        int64_t e = e0 + G::kKpp * j + ld_key;
        if (e > e_last) e = e_last;
        kreg[u][j] = *reinterpret_cast<const u32x4_t*>(keys + (size_t)(e + delta) * G::kKeyB + 16 * ld_chunk);
      }
      if constexpr (FP8) {
        int64_t e = e0 + li;
        if (e > e_last) e = e_last;
        sreg[u] = ksc[e + delta];
      }
      if constexpr (FP4) {
        int64_t e = e0 + li;
        if (e > e_last) e = e_last;
        sreg[u] = ksc4[(size_t)(e + delta) * (kD / 32) + lg];
      }
    }
  };
  KBatch kA, kB;
  SBatch sA, sB;
  if (nbatch > 0) load_batch(kA, sA, 0);
  if (nbatch > 1) load_batch(kB, sB, 1);
  __builtin_amdgcn_sched_barrier(0);

  // the per-head query scale (e4m3) folds into the head weight
  if constexpr (FP8) {
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      wr[ht][0] *= qs[ht].x; wr[ht][1] *= qs[ht].y; wr[ht][2] *= qs[ht].z; wr[ht][3] *= qs[ht].w;
    }
  }
  if (use_hist) {
    for (int i = tid; i < kTopkBins; i += 256) s_hist[i] = 0;
    lds_barrier();  // LDS only: the key loads in flight are not waited for
  }

  // LDS positions: where this lane writes its chunk of piece j, where it
  // reads its MFMA operand chunks
  char* tr = s_tr[w];
  int wr_off[G::kPieces];
#pragma unroll
  for (int j = 0; j < G::kPieces; ++j) wr_off[j] = G::lds_off(G::kKpp * j + ld_key, ld_chunk);
  constexpr int kReads = FP8 ? 2 : 4;
  int rd_off[kReads];
#pragma unroll
  for (int r = 0; r < kReads; ++r) rd_off[r] = G::lds_off(li, FP8 ? lg + 4 * r : 4 * r + lg);

  // score tiles u, u+1 of the batch in the transpose buffer (interleaved so
  // the two latency chains overlap)
  constexpr int kG = 2;
  auto score = [&](const KBatch& kcur, const SBatch& sreg, int bi, int u) __attribute__((always_inline)) {
    float part[kG];
#pragma unroll
    for (int g = 0; g < kG; ++g) part[g] = 0.f;
    if constexpr (FP4) {
      // the block scales of both operands enter the MFMA (per lane: the
      // query block's and the key block's E8M0 codes)
      f32x4_t c[HT][kG];
#pragma unroll
      for (int ht = 0; ht < HT; ++ht)
#pragma unroll
        for (int g = 0; g < kG; ++g) {
          const u32x4_t k4 = kcur[u + g][0];
          const i32x8_t kb = i32x8_t{(int)k4.x, (int)k4.y, (int)k4.z, (int)k4.w, 0, 0, 0, 0};
          c[ht][g] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(q8[ht], kb, f32x4_t{0.f, 0.f, 0.f, 0.f}, 4, 4,
                                                                      0, qsc[ht], 0, (int)sreg[u + g]);
        }
#pragma unroll
      for (int ht = 0; ht < HT; ++ht)
#pragma unroll
        for (int g = 0; g < kG; ++g)
#pragma unroll
          for (int r = 0; r < 4; ++r) part[g] += wr[ht][r] * relu(c[ht][g][r]);
    } else if constexpr (FP8) {
      i32x8_t kb[kG];
#pragma unroll
      for (int g = 0; g < kG; ++g) {
        const char* src = tr + (u + g) * G::kTileB;
        const uint4 v0 = *reinterpret_cast<const uint4*>(src + rd_off[0]);
        const uint4 v1 = *reinterpret_cast<const uint4*>(src + rd_off[1]);
        kb[g] = i32x8_t{(int)v0.x, (int)v0.y, (int)v0.z, (int)v0.w, (int)v1.x, (int)v1.y, (int)v1.z, (int)v1.w};
      }
      f32x4_t c[HT][kG];
#pragma unroll
      for (int ht = 0; ht < HT; ++ht)
#pragma unroll
        for (int g = 0; g < kG; ++g)
          c[ht][g] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(q8[ht], kb[g], f32x4_t{0.f, 0.f, 0.f, 0.f},
                                                                      0, 0, 0, 127, 0, 127);
#pragma unroll
      for (int ht = 0; ht < HT; ++ht)
#pragma unroll
        for (int g = 0; g < kG; ++g)
#pragma unroll
          for (int r = 0; r < 4; ++r) part[g] += wr[ht][r] * relu(c[ht][g][r]);
    } else {
      bf16x8_t kf[kG][4];
#pragma unroll
      for (int g = 0; g < kG; ++g)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          kf[g][ks] = *reinterpret_cast<const bf16x8_t*>(tr + (u + g) * G::kTileB + rd_off[ks]);
      f32x4_t c[HT][kG];
#pragma unroll
      for (int ht = 0; ht < HT; ++ht)
#pragma unroll
        for (int g = 0; g < kG; ++g) c[ht][g] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
#pragma unroll
          for (int g = 0; g < kG; ++g)
            c[ht][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qb[ht][ks], kf[g][ks], c[ht][g], 0, 0, 0);
#pragma unroll
      for (int ht = 0; ht < HT; ++ht)
#pragma unroll
        for (int g = 0; g < kG; ++g)
#pragma unroll
          for (int r = 0; r < 4; ++r) part[g] += wr[ht][r] * relu(c[ht][g][r]);
    }
#pragma unroll
    for (int g = 0; g < kG; ++g) {
      // head sum over the four lane groups: lanes l, l^16, l^32, l^48
      part[g] = lane_sum_xor16_32(part[g]);
      if (FP8) part[g] *= sreg[u + g];
      if (a.score_bf16) part[g] = round_bf16(part[g]);
      const int i = bi * kU + u + g;
      const int64_t e = (t0 + i) * 16 + li;
      if (e < nv_scan && i < n && lg == 0) {
        out[e] = part[g];
        if (use_hist) atomicAdd(&s_hist[f32_key(part[g]) >> kTopkShift], 1);
        if (fuse) s_sc[(w * per + i) * 16 + li] = part[g];
      }
    }
  };

  // transpose a batch through this wavefront's LDS buffer and score it; the
  // writes land before the reads (the wavefront's own LDS operations, in
  // order).  MXFP4 batches are already in operand layout.
  auto run_batch = [&](KBatch& kcur, SBatch& scur, int bi) __attribute__((always_inline)) {
    if constexpr (!FP4) {
#pragma unroll
      for (int u = 0; u < kU; ++u)
#pragma unroll
        for (int j = 0; j < G::kPieces; ++j)
          *reinterpret_cast<u32x4_t*>(tr + u * G::kTileB + wr_off[j]) = kcur[u][j];
    }
#pragma unroll
    for (int u = 0; u < kU; u += kG) score(kcur, scur, bi, u);
  };
  // two register batches alternate; loads are unconditional (past the run
  // they hit one cached row), so the compiler's wait bookkeeping sees the
  // same outstanding loads on every path and only waits for the batch that
  // is about to be used
  // batches bi, bi+1 are in flight when step bi starts; a register batch is
  // refilled (batch bi+2) as soon as its data has gone to LDS
  if (nbatch > 0) {
    for (int bi = 0; bi < nbatch; bi += 2) {
      run_batch(kA, sA, bi);
      load_batch(kA, sA, bi + 2);
      if (bi + 1 < nbatch) {
        run_batch(kB, sB, bi + 1);
        load_batch(kB, sB, bi + 3);
      }
    }
  }
  if (fold_wg) {
    // the step's compressor work for this sequence (the scan above was empty).
    // The new token's appends to the tail rings and the window ring need only
    // the step's inputs, and the tail slot they write (t mod R, with R > 2m)
    // is never a source of the fold: their loads go out first, together with
    // the fold's (one round trip for both), and their stores come last.  In
    // 16-byte chunks: the main streams, the indexer streams, the window row.
    const int nstr = f.overlap ? 4 : 2;
    const int slot_t = (int)(t % f.R);
    const int n_mc = nstr * f.c / 8, n_ic = 4 * kD / 8, n_ap = n_mc + n_ic + f.c / 8;
    constexpr int kAp = 2;  // chunks per thread: n_ap <= 4 * 512 / 8 + 64 + 64 = 384
    uint4 ap[kAp];
#pragma unroll
    for (int u = 0; u < kAp; ++u) {
      const int i = tid + 256 * u;
      const uint16_t* src = nullptr;
      if (i < n_mc)
        src = reinterpret_cast<const uint16_t*>(f.streams) + (size_t)b * nstr * f.c + 8 * i;
      else if (i < n_mc + n_ic)
        src = reinterpret_cast<const uint16_t*>(f.idx_streams) + (size_t)b * 4 * kD + 8 * (i - n_mc);
      else if (i < n_ap)
        src = reinterpret_cast<const uint16_t*>(f.x_new) + (size_t)b * f.c + 8 * (i - n_mc - n_ic);
      ap[u] = src ? *reinterpret_cast<const uint4*>(src) : uint4{0, 0, 0, 0};
    }
    auto store_appends = [&]() {
#pragma unroll
      for (int u = 0; u < kAp; ++u) {
        const int i = tid + 256 * u;
        uint16_t* dst = nullptr;
        if (i < n_mc) {
          const int sc = 8 * i / f.c, r = 8 * i % f.c;
          dst = reinterpret_cast<uint16_t*>(f.tail) + (((size_t)b * nstr + sc) * f.R + slot_t) * f.c + r;
        } else if (i < n_mc + n_ic) {
          const int j = 8 * (i - n_mc), sc = j / kD, r = j % kD;
          dst = reinterpret_cast<uint16_t*>(f.idx_tail) + (((size_t)b * 4 + sc) * f.R + slot_t) * kD + r;
        } else if (i < n_ap) {
          dst = reinterpret_cast<uint16_t*>(f.win_ring) + ((size_t)b * f.n_win + t % f.n_win) * f.c +
                8 * (i - n_mc - n_ic);
        }
        if (dst) *reinterpret_cast<uint4*>(dst) = ap[u];
      }
    };

    // bytes of one query vector, in 16-byte loads
    constexpr int kQB = FP4 ? kD / 2 : (FP8 ? kD : 2 * kD);
    constexpr int kV = kQB / 16;
    Soft* s_part = reinterpret_cast<Soft*>(&s_tr[0][0]);
    float* s_red = reinterpret_cast<float*>(s_part + 4 * 256);
    uint32_t* s_key = reinterpret_cast<uint32_t*>(s_red + 8);  // the stored new key (<= 256 B)
    const int64_t e = n_have;
    // the new entry's cache row (PG: through the block table; its load goes
    // out with the fold's sources)
    size_t frow = (size_t)b * a.E_cap + e;
    if constexpr (PG) frow = fold_now ? page_row(a.pg, b, e, a.E_cap) : 0;
    // the new key's score, as the scan computes it: sum_h w_h q_scale_h
    // ReLU(q_h . k), times the key scale (wave 0, lane = head; qv_reg holds
    // the lane's query row when pre, else it is loaded here)
    auto score_new_key = [&](float ks, const uint4* qv_reg, bool pre) {
      if (w != 0) return;
      float part = 0.f;
      if (l < H) {
        const uint4* qv = reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(a.q) +
                                                         ((size_t)row * H + l) * kQB);
        const uint4* kv4 = reinterpret_cast<const uint4*>(s_key);
        uint4 qr[kV];
#pragma unroll
        for (int j = 0; j < kV; ++j) qr[j] = pre ? qv_reg[j] : qv[j];
        float c = 0.f;
        if constexpr (FP4) {
          // per block of 32: the E2M1 products summed exactly, then both
          // block scales (as the scaled MFMA applies them)
          const uint32_t qs4 = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(a.q_scale) +
                                                                  ((size_t)row * H + l) * (kD / 32));
          const uint32_t ks4 = s_key[kD / 8];  // the four key scales after the 64 code bytes
#pragma unroll
          for (int j = 0; j < kV; ++j) {
            const uint4 kj = kv4[j];
            const uint32_t qw[4] = {qr[j].x, qr[j].y, qr[j].z, qr[j].w};
            const uint32_t kw[4] = {kj.x, kj.y, kj.z, kj.w};
            float blk = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
              for (int n = 0; n < 8; ++n)
                blk += e2m1_to_f32((qw[i] >> (4 * n)) & 15u) * e2m1_to_f32((kw[i] >> (4 * n)) & 15u);
            c += blk * e8m0_to_f32((qs4 >> (8 * j)) & 255u) * e8m0_to_f32((ks4 >> (8 * j)) & 255u);
          }
        } else {
#pragma unroll
        for (int j = 0; j < kV; ++j) {
          const uint4 kj = kv4[j];
          const uint32_t qw[4] = {qr[j].x, qr[j].y, qr[j].z, qr[j].w};
          const uint32_t kw[4] = {kj.x, kj.y, kj.z, kj.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if constexpr (FP8) {
              c += __builtin_amdgcn_cvt_f32_fp8((int)qw[i], 0) * __builtin_amdgcn_cvt_f32_fp8((int)kw[i], 0);
              c += __builtin_amdgcn_cvt_f32_fp8((int)qw[i], 1) * __builtin_amdgcn_cvt_f32_fp8((int)kw[i], 1);
              c += __builtin_amdgcn_cvt_f32_fp8((int)qw[i], 2) * __builtin_amdgcn_cvt_f32_fp8((int)kw[i], 2);
              c += __builtin_amdgcn_cvt_f32_fp8((int)qw[i], 3) * __builtin_amdgcn_cvt_f32_fp8((int)kw[i], 3);
            } else {
              c += __uint_as_float(qw[i] << 16) * __uint_as_float(kw[i] << 16);
              c += __uint_as_float(qw[i] & 0xffff0000u) * __uint_as_float(kw[i] & 0xffff0000u);
            }
          }
        }
        }
        part = FP8 ? a.w[(size_t)row * H + l] * reinterpret_cast<const float*>(a.q_scale)[(size_t)row * H + l] *
                         relu(c)
                   : a.w[(size_t)row * H + l] * relu(c);
      }
      part = wave_sum(part);
      if (FP8) part *= ks;
      if (a.score_bf16) part = round_bf16(part);
      if (l == 0) {
        out[e] = part;
        s_sc[0] = part;
        if (use_hist) s_hist[f32_key(part) >> kTopkShift] += 1;
      }
    };
    // the new indexer key (value iv of coordinate tid < kD) to its storage
    // format, into the cache and s_key; returns its scale (1 for bf16)
    auto store_key = [&](float iv) -> float {
      const size_t krow = frow;
      float ks = 1.f;
      if constexpr (FP4) {
        // blocks of 32 coordinates = lane groups of 32 of waves 0 and 1;
        // codes to the cache and to s_key (64 bytes), then the 4 scales
        uint32_t sc;
        const uint32_t code = mx_quantize_lane(tid < kD ? iv : 0.f, &sc);
        const uint32_t odd = __shfl_xor(code, 1, 64);
        if (tid < kD && (tid & 1) == 0) {
          const uint8_t byte = (uint8_t)(code | (odd << 4));
          reinterpret_cast<uint8_t*>(f.idx_cache)[krow * (kD / 2) + tid / 2] = byte;
          reinterpret_cast<uint8_t*>(s_key)[tid / 2] = byte;
        }
        if (tid < kD && (tid & 31) == 0) {
          reinterpret_cast<uint8_t*>(f.idx_scale)[krow * (kD / 32) + tid / 32] = (uint8_t)sc;
          reinterpret_cast<uint8_t*>(s_key)[kD / 2 + tid / 32] = (uint8_t)sc;
        }
      } else if constexpr (FP8) {
        float am = wave_max(tid < kD ? fabsf(iv) : 0.f);
        if (l == 0) s_red[w] = am;
        __syncthreads();
        am = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
        ks = am / 448.0f;
        if (!(ks > 0.f)) ks = 1.f;
        if (tid < kD) {
          const uint8_t code = f32_to_e4m3(iv / ks);
          reinterpret_cast<uint8_t*>(f.idx_cache)[krow * kD + tid] = code;
          reinterpret_cast<uint8_t*>(s_key)[tid] = code;
        }
        if (tid == 0) reinterpret_cast<float*>(f.idx_scale)[krow] = ks;
      } else {
        if (tid < kD) {
          const uint16_t v = f32_to_bf16(iv);
          reinterpret_cast<uint16_t*>(f.idx_cache)[krow * kD + tid] = v;
          reinterpret_cast<uint16_t*>(s_key)[tid] = v;
        }
      }
      __syncthreads();
      return ks;
    };
    if (fold_now && f.m <= kFastFoldM && f.c <= kFastFoldC) {
      // Every source of the block, for the main entry and the indexer key,
      // with its positional bias, staged in LDS by one round of loads
      // (kFastFoldM sources per branch, kFastFoldC coordinates at most: 24
      // KB in the transpose buffer, the main entry's biases (16 KB) in the
      // score buffer, of which this workgroup needs only its first slot, and
      // only after the fold), and the query rows the new key's score needs
      // loaded with them; then each thread folds whole coordinates.
      const int m = f.m, c = f.c, R = f.R;
      const bool use_bm = f.overlap && e > 0;  // the main entry's branch b (the previous block)
      const bool use_bi = e > 0;               // the indexer key always overlaps
      const int Sm = use_bm ? 2 * m : m, Si = use_bi ? 2 * m : m;
      constexpr int kS = 2 * kFastFoldM;
      static_assert(kS * kFastFoldC * 2 * 2 + kS * kD * 8 + 288 <= sizeof(s_tr), "fold staging fits");
      static_assert(kS * kFastFoldC <= kTopkFuseCap, "main biases fit the score buffer");
      uint16_t* mz = reinterpret_cast<uint16_t*>(&s_tr[0][0]);  // [kS][kFastFoldC] logits
      uint16_t* mx = mz + kS * kFastFoldC;                      // [kS][kFastFoldC] contents
      float* mb = s_sc;                                         // [kS][kFastFoldC] biases
      uint16_t* iz = mx + kS * kFastFoldC;                      // [kS][kD]
      uint16_t* ix = iz + kS * kD;
      float* ib = reinterpret_cast<float*>(ix + kS * kD);
      s_red = ib + kS * kD;
      s_key = reinterpret_cast<uint32_t*>(s_red + 8);
      const int mstr = f.overlap ? 4 : 2;
      const uint16_t* mtail = reinterpret_cast<const uint16_t*>(f.tail) + (size_t)b * mstr * R * c;
      const uint16_t* mio = reinterpret_cast<const uint16_t*>(f.streams) + (size_t)b * mstr * c;
      const uint16_t* itail = reinterpret_cast<const uint16_t*>(f.idx_tail) + (size_t)b * 4 * R * kD;
      const uint16_t* iio = reinterpret_cast<const uint16_t*>(f.idx_streams) + (size_t)b * 4 * kD;
      // row of source j of a block's fold in stream (0: content, 1: logit):
      // j < m is token e m + j of branch a, else token (e-1) m + j - m of
      // branch b; the new token t comes from the step's inputs
      auto src = [&](const uint16_t* tail, const uint16_t* io, int width, int j, int logit) -> const uint16_t* {
        const int stream = (j < m ? 0 : 2) + logit;
        const int64_t tok = j < m ? e * m + j : (e - 1) * m + (j - m);
        if (tok == t) return io + (size_t)stream * width;
        return tail + ((size_t)stream * R + (size_t)(tok % R)) * width;
      };
      auto bias = [&](const float* ba, const float* bb, int width, int j) -> const float* {
        const float* p = j < m ? ba : bb;
        return p ? p + (size_t)(j < m ? j : j - m) * width : nullptr;
      };
      constexpr int kMC = kS * kFastFoldC / 8 / 256;  // 16-byte chunks per thread (logits, contents)
      constexpr int kMB = kS * kFastFoldC / 4 / 256;  // (biases)
      uint4 rz[kMC], rx[kMC], rb[kMB], riz, rix, rib;
      const int cpr = c / 8, bpr = c / 4;  // 16-byte chunks per main row (bf16, f32)
#pragma unroll
      for (int u = 0; u < kMC; ++u) {
        const int i = tid + 256 * u, j = i / cpr, cc = i % cpr;
        rz[u] = rx[u] = uint4{0, 0, 0, 0};
        if (j < Sm) {
          rz[u] = *reinterpret_cast<const uint4*>(src(mtail, mio, c, j, 1) + 8 * cc);
          rx[u] = *reinterpret_cast<const uint4*>(src(mtail, mio, c, j, 0) + 8 * cc);
        }
      }
#pragma unroll
      for (int u = 0; u < kMB; ++u) {
        const int i = tid + 256 * u, j = i / bpr, cc = i % bpr;
        const float* bp = j < Sm ? bias(f.bias_a, f.bias_b, c, j) : nullptr;
        rb[u] = bp ? *reinterpret_cast<const uint4*>(bp + 4 * cc) : uint4{0, 0, 0, 0};
      }
      {
        const int j = tid / (kD / 8), cc = tid % (kD / 8);
        riz = rix = uint4{0, 0, 0, 0};
        if (j < Si) {
          riz = *reinterpret_cast<const uint4*>(src(itail, iio, kD, j, 1) + 8 * cc);
          rix = *reinterpret_cast<const uint4*>(src(itail, iio, kD, j, 0) + 8 * cc);
        }
        const int jb = tid / (kD / 4), cb = tid % (kD / 4);
        const float* bp = jb < Si ? bias(f.ibias_a, f.ibias_b, kD, jb) : nullptr;
        rib = bp ? *reinterpret_cast<const uint4*>(bp + 4 * cb) : uint4{0, 0, 0, 0};
      }
      uint4 qreg[kV];
      if (w == 0 && l < H) {
        const uint4* qv = reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(a.q) +
                                                         ((size_t)row * H + l) * kQB);
#pragma unroll
        for (int j = 0; j < kV; ++j) qreg[j] = qv[j];
      }
      // to LDS (row j at j * width)
#pragma unroll
      for (int u = 0; u < kMC; ++u) {
        const int i = tid + 256 * u, j = i / cpr, cc = i % cpr;
        if (j < Sm) {
          *reinterpret_cast<uint4*>(mz + j * kFastFoldC + 8 * cc) = rz[u];
          *reinterpret_cast<uint4*>(mx + j * kFastFoldC + 8 * cc) = rx[u];
        }
      }
#pragma unroll
      for (int u = 0; u < kMB; ++u) {
        const int i = tid + 256 * u, j = i / bpr, cc = i % bpr;
        if (j < Sm) *reinterpret_cast<uint4*>(mb + j * kFastFoldC + 4 * cc) = rb[u];
      }
      {
        const int j = tid / (kD / 8), cc = tid % (kD / 8);
        if (j < Si) {
          *reinterpret_cast<uint4*>(iz + j * kD + 8 * cc) = riz;
          *reinterpret_cast<uint4*>(ix + j * kD + 8 * cc) = rix;
        }
        const int jb = tid / (kD / 4), cb = tid % (kD / 4);
        if (jb < Si) *reinterpret_cast<uint4*>(ib + jb * kD + 4 * cb) = rib;
      }
      __syncthreads();
      // one coordinate per thread: a softmax over the sources' logits
      // (+ biases) weights their contents
      auto fold_coord = [&](const uint16_t* zr, const uint16_t* xr, const float* br, int width, int S, int r) {
        float mxv = -INFINITY;
#pragma unroll
        for (int j = 0; j < kS; ++j)
          if (j < S) mxv = fmaxf(mxv, bf16_to_f32(zr[j * width + r]) + br[j * width + r]);
        float lsum = 0.f, acc = 0.f;
#pragma unroll
        for (int j = 0; j < kS; ++j) {
          if (j < S) {
            const float ex = __expf(bf16_to_f32(zr[j * width + r]) + br[j * width + r] - mxv);
            lsum += ex;
            acc += ex * bf16_to_f32(xr[j * width + r]);
          }
        }
        return acc / lsum;
      };
      const float iv = tid < kD ? fold_coord(iz, ix, ib, kD, Si, tid) : 0.f;
      const float ks = store_key(iv);
      for (int r = tid; r < c; r += 256)
        reinterpret_cast<uint16_t*>(f.kv_cache)[frow * c + r] =
            f32_to_bf16(fold_coord(mz, mx, mb, kFastFoldC, Sm, r));
      __syncthreads();  // every read of the biases in s_sc is done
      score_new_key(ks, qreg, true);
    } else if (fold_now) {
      // indexer key: fold, quantize, store
      const bf16* itail = reinterpret_cast<const bf16*>(f.idx_tail) + (size_t)b * 4 * f.R * kD;
      const bf16* iio = reinterpret_cast<const bf16*>(f.idx_streams) + (size_t)b * 4 * kD;
      const float iv = fold_job<bf16>(itail, iio, kD, 0, kD, f.m, f.R, t, e, e > 0, f.ibias_a, f.ibias_b, s_part);
      const float ks = store_key(iv);
      score_new_key(ks, nullptr, false);
      // main entry: two halves of the coordinates
      const bf16* mtail = reinterpret_cast<const bf16*>(f.tail) + (size_t)b * (f.overlap ? 4 : 2) * f.R * f.c;
      const bf16* mio = reinterpret_cast<const bf16*>(f.streams) + (size_t)b * (f.overlap ? 4 : 2) * f.c;
      for (int r0 = 0; r0 < f.c; r0 += 256) {
        const int W = f.c - r0 < 256 ? f.c - r0 : 256;
        const float v = fold_job<bf16>(mtail, mio, f.c, r0, W, f.m, f.R, t, e, f.overlap && e > 0, f.bias_a,
                                       f.bias_b, s_part);
        if (tid < W) reinterpret_cast<uint16_t*>(f.kv_cache)[frow * f.c + r0 + tid] = f32_to_bf16(v);
      }
    }
    store_appends();
  }
  if (use_hist) {
    __syncthreads();
    int* gh = ws.hist + (size_t)row * kTopkBins;
    for (int i = tid; i < kTopkBins; i += 256) {
      const int v = s_hist[i];
      if (v) atomicAdd(&gh[i], v);
    }
  }
  const bool select = fuse && nv > a.k;  // nv <= k: every visible entry is selected
  if (!select && !fold_now) return;

  // ---- fused collection.  Arrive on the row counter once this workgroup's
  // histogram atomics (and fold stores) have completed (device scope).
  int* slot = ws.ctr + (size_t)row * 4;  // [2] failure flag, [3] published threshold bin
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) s_misc[15] = atomicAdd(&ws.sync[row], 1u) == gridDim.x - 1;
  __syncthreads();
  // the last to arrive: every workgroup of the row has read the old count
  if (s_misc[15] && fold_now && tid == 0)
    __hip_atomic_store(f.n_entries + b, n_have + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (!select) return;
  int b1, above;
  if (s_misc[15]) {
    // last of the row: the histogram is complete; read it device-coherently,
    // all eight loads of a thread in flight together (bins in descending
    // order over the threads, as find_bin_counts takes them)
    const int* gh = ws.hist + (size_t)row * kTopkBins + (kTopkBins - 1) - 8 * tid;
    int c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = __hip_atomic_load(gh - i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    find_bin_counts<256>(c, a.k, s_misc, s_misc + 8, &b1, &above);
    if (tid == 0)
      __hip_atomic_store(slot + 3, (1 << 30) | (above << 11) | b1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    if (tid == 0) {
      // four polls in flight, issued about 0.05 us apart: the publication
      // is seen about one round trip after it lands, not one round trip
      // plus a poll period
      int v = 0;
      for (int it = 0; it < wait_polls / 4 && v == 0; ++it) {
        const int v0 = __hip_atomic_load(slot + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_s_sleep(2);
        const int v1 = __hip_atomic_load(slot + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_s_sleep(2);
        const int v2 = __hip_atomic_load(slot + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_s_sleep(2);
        const int v3 = __hip_atomic_load(slot + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        v = v0 ? v0 : (v1 ? v1 : (v2 ? v2 : v3));
      }
      s_misc[14] = v;
    }
    __syncthreads();
    const int v = s_misc[14];
    if (v == 0) {  // not published in time: the row falls back to a scan of its scores
      if (tid == 0) atomicOr(slot + 2, 1);
      return;
    }
    b1 = v & 2047;
    above = (v >> 11) & 4095;
  }
  int64_t e_first = (int64_t)blockIdx.x * 4 * per * 16;
  int n_ent = (int)(nv_scan - e_first < 0 ? 0 : nv_scan - e_first);
  if (n_ent > 4 * per * 16) n_ent = 4 * (int)per * 16;
  if (fold_wg) {  // its one entry, the new one
    e_first = n_have;
    n_ent = fold_now ? 1 : 0;
  }
  int4* info = ws.wg_info + (size_t)row * kTopkMaxWgRow + blockIdx.x;
  // contiguous runs per thread keep the lists in entry order; a run is a
  // multiple of 4 entries, read once as 16-byte vectors into registers
  constexpr int kRun = kTopkFuseCap / 256;  // entries per thread, at most
  const int cpt = ((n_ent + 255) / 256 + 3) & ~3;
  const int i0 = tid * cpt;
  uint32_t key[kRun];
  int cnt = 0;  // certain winners in the low half, candidates in the high half
#pragma unroll
  for (int v = 0; v < kRun / 4; ++v) {
    float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
    if (4 * v < cpt && i0 + 4 * v < n_ent) f = *reinterpret_cast<const float4*>(s_sc + i0 + 4 * v);
    const float fv[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = 4 * v + u;
      key[i] = f32_key(fv[u]);
      const int bin = (int)(key[i] >> kTopkShift);
      if (i < cpt && i0 + i < n_ent) cnt += (bin > b1 ? 1 : 0) + (bin == b1 ? 1 << 16 : 0);
    }
  }
  int total;
  const int off = block_excl_scan<256>(cnt, s_misc, &total);
  int os = off & 0xffff, oc = off >> 16;
  const size_t list_off = (size_t)row * ws.list_len + (size_t)blockIdx.x * ws.list_stride;
  int* lsure = ws.lsure + list_off;
  uint2* lcand = ws.lcand + list_off;
#pragma unroll
  for (int i = 0; i < kRun; ++i) {
    const bool in = i < cpt && i0 + i < n_ent;
    const int bin = (int)(key[i] >> kTopkShift);
    if (in && bin > b1) lsure[os++] = (int)e_first + i0 + i;
    if (in && bin == b1) lcand[oc++] = make_uint2(key[i], (uint32_t)(e_first + i0 + i));
  }
  if (tid == 0) *info = make_int4(total & 0xffff, (unsigned)total >> 16, (int)e_first, 0);
}

bool index_mfma_supported(const IndexArgs& a) {
  return (a.idx_dtype == BF16 || a.idx_dtype == E4M3 || a.idx_dtype == MXFP4) && a.d_I == kD && a.H_I % 16 == 0 &&
         a.H_I <= 64;
}

// workgroups that fit on the device at once for a kernel of 256 threads
template <typename K>
static int resident_wgs(K kernel) {
  int dev = 0, n_cu = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 1024;
  if (hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 1024;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, 0) != hipSuccess || per_cu < 1)
    per_cu = 1;
  return n_cu * per_cu;
}

// Grid of the scan: one round of resident workgroups (the scan is a single
// pass over the keys), at most one workgroup per 16 tiles of a row.  Fused
// collection when the grid fits on the device at once and a workgroup's
// scores (4 waves x per tiles, for the largest visible count E_cap) fit in
// its LDS; with a fold, the last workgroup of each row is the fold
// workgroup.
struct ScorerPlan {
  int per_row, fuse, list_stride;
};
static ScorerPlan scorer_plan(const IndexArgs& a, int resident, int use_hist, int allow_fuse, int with_fold) {
  const int rows = a.B * a.Tq;
  int per_row = resident / rows;
  const int max_wg = (int)((((int64_t)a.E_cap + 15) / 16 + 15) / 16) + with_fold;
  if (per_row > max_wg) per_row = max_wg;
  if (per_row < 1 + with_fold) per_row = 1 + with_fold;
  const int scan_wg = per_row - with_fold;
  const int64_t per = ((int64_t)a.E_cap + 15) / 16 / ((int64_t)scan_wg * 4) + 1;
  const int fuse = allow_fuse && use_hist && per_row * rows <= resident && per_row <= kTopkMaxWgRow &&
                   4 * per * 16 <= kTopkFuseCap && (int64_t)per_row * 4 * per * 16 <= topk_list_len(a.E_cap);
  return ScorerPlan{per_row, fuse, (int)(4 * per * 16)};
}

// per device: the grid of the scan is sized to the device's resident count
// (of the instantiation that runs: contiguous or paged keys)
template <int FMT, int HT, int PG>
static int scorer_resident() {
  static std::atomic<int> resident[kMaxDevices];
  const int dev = current_device();
  if (dev < 0) return resident_wgs(index_score_mfma_kernel<FMT, HT, PG>);
  int r = resident[dev].load(std::memory_order_relaxed);
  if (!r) {
    r = resident_wgs(index_score_mfma_kernel<FMT, HT, PG>);
    resident[dev].store(r, std::memory_order_relaxed);
  }
  return r;
}

template <int FMT, int HT, int PG>
static hipError_t launch_scorer(const IndexArgs& a, TopkWs& ws, int use_hist, int allow_fuse,
                                int* n_wg_fused, const FoldArgs* fold, hipStream_t s) {
  const int with_fold = fold ? 1 : 0;
  const ScorerPlan p = scorer_plan(a, scorer_resident<FMT, HT, PG>(), use_hist, allow_fuse && ws.sync != nullptr,
                                   with_fold);
  if (with_fold && !p.fuse) return hipErrorInvalidValue;  // the caller checks index_fold_fusable first
  *n_wg_fused = p.fuse ? p.per_row : 0;
  ws.list_stride = p.list_stride;  // (also read by the resolve kernel)
  FoldArgs f = fold ? *fold : FoldArgs{};
  dim3 grid(p.per_row, a.B * a.Tq), block(256);
  CSA_LAUNCH("index_score_mfma", (index_score_mfma_kernel<FMT, HT, PG>), grid, block, 0, s, a, ws, use_hist, p.fuse,
             f, with_fold, fused_wait_polls());
  return hipGetLastError();
}

template <int FMT, int PG>
static int resident_for(int HT) {
  if (HT == 4) return scorer_resident<FMT, 4, PG>();
  if (HT == 3) return scorer_resident<FMT, 3, PG>();
  if (HT == 2) return scorer_resident<FMT, 2, PG>();
  return scorer_resident<FMT, 1, PG>();
}

static int scan_format(int idx_dtype) { return idx_dtype == MXFP4 ? 2 : (idx_dtype == E4M3 ? 1 : 0); }

// paged keys: a 16-entry tile within one page (>= 16 entries per page) and
// a wave's run within 64 pages (the run of the scan's grid for E_cap)
static int resident_of(const IndexArgs& a) {
  const int fmt = scan_format(a.idx_dtype), HT = a.H_I / 16;
  if (a.pg.table)
    return fmt == 2 ? resident_for<2, 1>(HT) : (fmt == 1 ? resident_for<1, 1>(HT) : resident_for<0, 1>(HT));
  return fmt == 2 ? resident_for<2, 0>(HT) : (fmt == 1 ? resident_for<1, 0>(HT) : resident_for<0, 0>(HT));
}

// paged keys: a 16-entry tile within one page (>= 16 entries per page) and
// a wave's run within 64 pages (the run of the scan's grid for E_cap, with
// or without the fold workgroup)
static bool pages_fit(const IndexArgs& a, int with_fold) {
  if (!a.pg.table) return true;
  if (a.pg.shift < 4) return false;
  const ScorerPlan p = scorer_plan(a, resident_of(a), 1, 1, with_fold);
  const int64_t ntile = ((int64_t)a.E_cap + 15) / 16, nwaves = (int64_t)(p.per_row - with_fold) * 4;
  const int64_t per = (ntile + nwaves - 1) / nwaves;
  return ((per * 16) >> a.pg.shift) + 2 <= 64;
}

bool index_mfma_pages_fit(const IndexArgs& a) { return pages_fit(a, 0); }

bool index_fold_fusable(const IndexArgs& a, const FoldArgs& f, bool split) {
  if (!split || !index_mfma_supported(a) || a.Tq != 1 || f.B != a.B || f.dtype != BF16 || f.kv_fmt ||
      f.idx_dtype != a.idx_dtype ||
      f.d_I != kD || a.n_add != 0 || !pages_fit(a, 1))
    return false;
  return scorer_plan(a, resident_of(a), 1, 1, 1).fuse != 0;
}

template <int FMT, int PG>
static hipError_t launch_scorer_fmt(const IndexArgs& a, TopkWs& ws, int use_hist, int allow_fuse,
                                    int* n_wg_fused, const FoldArgs* fold, hipStream_t s) {
  const int HT = a.H_I / 16;
  if (HT == 4) return launch_scorer<FMT, 4, PG>(a, ws, use_hist, allow_fuse, n_wg_fused, fold, s);
  if (HT == 3) return launch_scorer<FMT, 3, PG>(a, ws, use_hist, allow_fuse, n_wg_fused, fold, s);
  if (HT == 2) return launch_scorer<FMT, 2, PG>(a, ws, use_hist, allow_fuse, n_wg_fused, fold, s);
  return launch_scorer<FMT, 1, PG>(a, ws, use_hist, allow_fuse, n_wg_fused, fold, s);
}

template <int PG>
static hipError_t launch_scorer_pg(const IndexArgs& a, TopkWs& ws, int use_hist, int allow_fuse,
                                   int* n_wg_fused, const FoldArgs* fold, hipStream_t s) {
  const int fmt = scan_format(a.idx_dtype);
  if (fmt == 2) return launch_scorer_fmt<2, PG>(a, ws, use_hist, allow_fuse, n_wg_fused, fold, s);
  if (fmt == 1) return launch_scorer_fmt<1, PG>(a, ws, use_hist, allow_fuse, n_wg_fused, fold, s);
  return launch_scorer_fmt<0, PG>(a, ws, use_hist, allow_fuse, n_wg_fused, fold, s);
}

hipError_t launch_index_score_mfma(const IndexArgs& a, TopkWs& ws, int use_hist, int allow_fuse,
                                   int* n_wg_fused, const FoldArgs* fold, hipStream_t s) {
  if (a.pg.table) return launch_scorer_pg<1>(a, ws, use_hist, allow_fuse, n_wg_fused, fold, s);
  return launch_scorer_pg<0>(a, ws, use_hist, allow_fuse, n_wg_fused, fold, s);
}

}  // namespace csa
