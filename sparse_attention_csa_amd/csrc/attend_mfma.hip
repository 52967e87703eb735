// Dense (HCA) shared-KV attention on MFMA (bf16, entry dim 512): rows a5 +
// a6 of the hot path.
//
// What it computes is the generic kernel's result: for a query at position t
// and every head h, one softmax over all visible compressed entries and the
// window rows, with exp(sink_h) in the denominator ("DeepSeek-V4" book ch. 6
// "Shared key-value MQA", ch. 7 "The sliding window" and "Attention sinks").
// Every row is both key and value.
//
// Work split.  A workgroup (4 wavefronts, one per SIMD, the whole register
// file) owns one query, 64 heads (16 per wavefront) and a contiguous range of
// its rows ("split"); the splits of one query are merged by
// attend_merge_kernel with the online-softmax rule.  Every wavefront consumes
// every row of a tile, so a row crosses HBM / L2 into LDS once per split, not
// once per head group.  Row tiles of 32 rows (32 KB) are fetched into LDS by
// direct global-to-LDS DMA (one 1 KB row per wave instruction) into a ring of
// four slots: while tile j+1 is scored and tile j multiplied into the output,
// tiles j+2 and j+3 are in flight.
//
// Tied K = V on MFMA.  The score product is computed transposed,
//   S^T[rows x heads] = K[rows x d] . Q^T[d x heads]   (v_mfma 16x16x32 bf16),
// with Q^T held in registers and K read row-major from LDS.  The accumulator
// layout of S^T (lane = head, 4 consecutive rows per lane group) is, after
// exp2 and a bf16 cast, the B operand of
//   O^T[d x heads] += V^T[d x rows] . P^T[rows x heads]  (16x16x32 bf16)
// once the 32 reduction slots of a row pair (two 16-row blocks) are permuted
// consistently: slot 8g+i is row 4g+i of the first block for i < 4 and of
// the second for i >= 4.  V^T comes from the same LDS tile through the gfx950
// transpose read (ds_read_b64_tr_b16), whose per-lane addresses implement
// that permutation.  Softmax runs in base 2.
//
// Decode with the step's fold inside (fold_mode): the splits cover the
// entries that existed before the step and the window rows but the query's
// own token.  Split s of head group 0 also folds coordinates
// [s cs, s cs + cs) of the entry that the block ending at the query position
// completes: its sources, query slice and token slice arrive by DMA in the
// ring slot not yet in use, the fold runs before the row loop (nothing of it
// stays live across the loop), stores its slice of the entry, writes its
// share of q_h . entry and q_h . token for every head to its own slot of
// fold_s and appends its share of the token to the tail and window rings.
// The merge kernel then sums the slices' shares in slice order (the same
// order on every run: no atomics in the result path), adds the new entry and
// the query's own token as two more rows, weights exp2(scale q . x - M), and
// publishes the entry count.

#include <type_traits>

#include "fold.h"
#include "kernels.h"
#include "mfma_tile.h"

namespace csa {

using namespace tile;

namespace {

constexpr int kHW = 64;                // heads per workgroup (16 per wavefront)
constexpr int kTN = 32;                // rows per LDS tile
constexpr int kRing = 4;               // LDS tile slots: two tiles in use (scores, P.V), two in flight
constexpr int kRowsPerWave = kTN / 4;  // DMA instructions per wave and tile
constexpr int kFoldS = 16;             // fold slice: sources per thread (at most)
constexpr int kFoldRowsLess = 64;      // rows a folding split gives up to the others
constexpr int kFoldSlots = 64;         // fold slices at most (c / 8): one fold_s slot each
constexpr int kPgSplit = 4096;         // paged cache: page ids of one split's rows in LDS (at most;
                                       // pages past them are read from the table)

}  // namespace

// 1-D grid: block L runs on XCD L % 8; the n_hg head groups of one (query,
// split) are blocks L, L + 8, ... so they share that XCD's L2.
// DEROT: the output's rotary coordinates are rotated back by the query
// position (norm_rope); FOLD: the decode fold runs inside (fold_mode); PG:
// the cache is paged (the split's page ids are read into LDS first); SP:
// the compressed rows are a query's selected entries (sparse attention over
// a top-k list: the split's cache rows are read into LDS first, so the 64
// heads of a workgroup share one gather of each row).  Separate
// instantiations keep the code of one out of the others' register
// allocation (the row loop's schedule depends on it).
template <int DEROT, int FOLD, int PG, int SP>
__global__ __launch_bounds__(256, 1) void attend_mfma_kernel(AttendArgs a, int n_split, int rows_per_split) {
  __shared__ __attribute__((aligned(1024))) char tiles[kRing][kTN * kRowB];
  // PG: page ids of the split's cache rows; SP: the split's selected
  // entries' cache rows (-1: an id outside the cache, masked)
  __shared__ int32_t s_pg[(PG || SP) ? kPgSplit : 1];
  __shared__ uint32_t rvalid[kRing][kTN / 4];  // byte r % 4 of word r / 4: row r is a real row
  __shared__ int s_restart;                // a wavefront asks the split to be recomputed
  __shared__ bf16x8_t s_p[2][4][64];       // P^T operands of a tile (two buffers), one block of 16 heads per wavefront
  __shared__ float s_scale[kHW];           // output scale per head
  __shared__ Soft s_fpart[4][64];          // fold: per-wavefront partial states of <= 64 coordinates
  __shared__ float s_fnew[64];             // fold: the new entry's coordinates (bf16-rounded)
  __shared__ uint4 s_fapp[24];             // fold: x_new, stream 0, stream 1 slices (<= 64 coordinates each)

  const int n_hg = a.H / kHW;
  const int L = blockIdx.x;
  const int xcd = L & 7, kk = L >> 3;
  const int hg = kk % n_hg;
  const int rest = (kk / n_hg) * 8 + xcd;
  const int split = rest % n_split, qrow = rest / n_split;
  if (qrow >= a.B * a.Tq) return;

  const int b = qrow / a.Tq;
  const int tid = threadIdx.x, l = tid & 63, li = l & 15, lg = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = a.H;
  const int h0 = hg * kHW + 16 * w;  // this wavefront's first head

  // The position, entry count and window base (scalar loads) are requested
  // first.  The first tile's rows are usually cache entries whose addresses
  // need none of them, so its DMAs go out before they return (checked
  // below, reissued in the rare case).  (Unconditional loads: an absent
  // optional array is replaced by a valid dummy address and the value
  // discarded, so the three loads are in flight together instead of one
  // branch and wait each.)
  const int64_t* dummy64 = reinterpret_cast<const int64_t*>(a.kv);
  const int64_t t_ld = (a.q_pos ? a.q_pos + qrow : dummy64)[0];
  const int64_t w_ld = (a.win_pos0 ? a.win_pos0 + b : dummy64)[0];
  const int32_t cnt = SP ? a.topk_cnt[qrow] : a.n_entries[b];
  // row range of the split: with the fold inside, the first fold_nsplit
  // splits (the ones that fold) take fold_rows rows each, the rest
  // rows_per_split, so that the fold's time is balanced by fewer rows
  const int n_fs = a.fold_mode ? a.fold_nsplit : 0;
  const int rows_here = split < n_fs ? a.fold_rows : rows_per_split;
  const int r_begin = split < n_fs ? split * a.fold_rows : n_fs * a.fold_rows + (split - n_fs) * rows_per_split;
  const uint16_t* kv = reinterpret_cast<const uint16_t*>(a.kv) + (PG ? 0 : (size_t)b * a.E_cap * kC);

  // Wave w fetches rows kRowsPerWave * w .. of a tile; every wave reads all
  // rows.  Lane i (mod kRowsPerWave) computes the source of row
  // kRowsPerWave * w + i without branches; each DMA then takes its row's
  // address from that lane (two lane reads) and a per-lane chunk offset
  // fixed for the kernel.
  static_assert(kRowsPerWave == 8, "row validity words below");
  int dofs[kRowsPerWave];  // element offset of this lane's 16-byte chunk, per row
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) dofs[i] = 8 * (l ^ swz((kRowsPerWave * w + i) & 15));
  auto dma_rows = [&](const uint16_t* src, int buf) {
    const uintptr_t sp = reinterpret_cast<uintptr_t>(src);
    const uint32_t s_lo = (uint32_t)sp, s_hi = (uint32_t)(sp >> 32);
    uint32_t lds0 = lds_addr(tiles[buf]) + kRowsPerWave * w * kRowB;
    // (PG: the page-id reads before it leave the compiler unsure that the
    // slot address is uniform; it is)
    if constexpr (PG || SP) lds0 = __builtin_amdgcn_readfirstlane(lds0);
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      // (readlane returns int: widen through uint32_t, no sign extension)
      const uint64_t ri = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(s_hi, i) << 32) |
                          (uint64_t)(uint32_t)__builtin_amdgcn_readlane(s_lo, i);
      dma16_m0(reinterpret_cast<const uint16_t*>(ri) + dofs[i], lds0 + i * kRowB);
    }
  };
  // speculative: the first tile read as cache entries (in the cache
  // buffer, so in bounds whatever the count turns out to be), before
  // anything else
  const bool spec = !PG && !SP && r_begin + kTN <= a.E_cap;
  if (spec) dma_rows(kv + (size_t)(r_begin + kRowsPerWave * w + (l & (kRowsPerWave - 1))) * kC, 0);
  // Q^T operands for this wavefront's 16 heads: lane (head li, d group lg).
  // They are requested after the first tile's DMAs and before the
  // position, entry count and window base (scalar loads); the query loads
  // and the first tile are awaited together before the row loop, which the
  // later tiles' DMAs do not hold up.
  bf16x8_t qf[16];
  {
    const uint16_t* q = reinterpret_cast<const uint16_t*>(a.q) + ((size_t)qrow * H + h0 + li) * kC + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) qf[ks] = *reinterpret_cast<const bf16x8_t*>(q + 32 * ks);
  }
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);  // the scalars
  __asm__ __volatile__("" ::"s"(t_ld), "s"(w_ld), "s"(cnt));
  const int64_t t = a.q_pos ? t_ld : a.q_pos0 + qrow % a.Tq;
  const int64_t wpos0 = a.win_pos0 ? w_ld : a.win_pos0_const;
  const int64_t lim = vis_limit(t, a.m, a.vis);
  const int64_t have = (int64_t)cnt + a.n_add;
  int64_t n_c = lim < have ? lim : have;
  if (n_c > a.E_cap) n_c = a.E_cap;
  if (n_c < 0) n_c = 0;
  if constexpr (SP) n_c = cnt < 0 ? 0 : (cnt > a.k ? a.k : cnt);  // the selection (visible entries only)
  const int64_t n_w = (t + 1) < a.n_win ? (t + 1) : a.n_win;
  // fold_mode: the query's own token is not in the window ring yet; the
  // merge adds it as a row of its own
  const int64_t n_rows = n_c + n_w - (a.fold_mode ? 1 : 0);
  const int r_end = (int)((int64_t)r_begin + rows_here < n_rows ? r_begin + rows_here : n_rows);
  const int nc32 = (int)n_c;
  const uint16_t* win = reinterpret_cast<const uint16_t*>(a.win) + (size_t)b * a.W_cap * kC;
  const float sc2 = a.scale * kLog2e;
  // ring row of the first window position; later window rows follow with
  // one conditional wrap (n_win <= W_cap).  32-bit remainder when the
  // offset fits (always, for positions below 2^31).
  const int64_t wofs = t - n_w + 1 - wpos0;
  int wbase;
  if (wofs >= 0 && wofs < 0x7fffffff) {
    wbase = (int)((uint32_t)wofs % (uint32_t)a.W_cap);
  } else {
    int64_t wb = wofs % a.W_cap;
    if (wb < 0) wb += a.W_cap;
    wbase = (int)wb;
  }
  const int wcap = a.W_cap;
  // the query's own window row: always present, the source of padding rows
  // (their logits are masked)
  int own = wbase + (int)n_w - 1;
  if (own >= wcap) own -= wcap;
  const uint16_t* pad_row = win + (size_t)own * kC;

  // ---- fold slice (fold_mode, head group 0): coordinates [fr0, fr0 + fW)
  // of entry cnt, completed by the block ending at t (stored only if it is
  // the next entry: fold_now), this slice's share of q_h . entry and
  // q_h . token, and the token's share of the rings.  Its inputs come by DMA
  // into LDS with the first tiles (ring slot kRing - 1 and the P^T buffer
  // are unused until the row loop starts), so nothing of it is live during
  // the loop.
  const int fcs = a.fold_cs, fr0 = split * fcs;
  const int fW = (FOLD && a.fold_mode && hg == 0) ? (a.c - fr0 < 0 ? 0 : (a.c - fr0 < fcs ? a.c - fr0 : fcs)) : 0;
  const bool fold_now = fW > 0 && lim == (int64_t)cnt + 1 && cnt < a.E_cap;
  // the new entry's cache row (PG: through the block table)
  size_t frow = (size_t)b * a.E_cap + cnt;
  if constexpr (PG && FOLD) frow = fold_now ? page_row(a.pg, b, cnt, a.E_cap) : 0;
  const FoldArgs& F = a.fold;
  const int fch = fW / 8;                                  // 16-byte chunks per slice row (bf16)
  char* const fz_l = tiles[kRing - 1];                     // [m][fW] bf16: stream 1 (logits)
  char* const fx_l = fz_l + (size_t)F.m * fW * 2;          // [m][fW] bf16: stream 0 (values)
  char* const fb_l = fx_l + (size_t)F.m * fW * 2;          // [m][fW] f32: positional bias
  char* const fq_l = reinterpret_cast<char*>(&s_p[0][0][0]);  // [H][fW] bf16: query slice
  char* const fa_l = reinterpret_cast<char*>(s_fapp);      // [3][fW] bf16: x_new, streams 0, 1
  const uint16_t* const fio = reinterpret_cast<const uint16_t*>(F.streams) + (size_t)b * 2 * a.c;
  if (fW > 0) {
    // instruction k of a region moves its 16-byte chunks 64k .. 64k + 63,
    // one per lane, to LDS bytes 1024k ..; wavefront k % 4 issues it
    auto region = [&](int nq, char* dst, auto addr) {
      const int nk = (nq + 63) / 64;
      for (int k = w; k < nk; k += 4) {
        const int qq = 64 * k + l;
        if (qq < nq) dma16_m0(addr(qq), lds_addr(dst + 1024 * k));
      }
    };
    if (fold_now) {
      const int64_t p0 = (int64_t)cnt * F.m;  // first source token
      const int slot0 = p0 < 0x7fffffff ? (int)((uint32_t)p0 % (uint32_t)F.R) : (int)(p0 % F.R);
      const uint16_t* tl = reinterpret_cast<const uint16_t*>(F.tail) + (size_t)b * 2 * F.R * a.c;
      auto src = [&](int qq, int stream) -> const void* {
        const int j = qq / fch, cc = fr0 + 8 * (qq % fch);
        int slot = slot0 + j;
        if (slot >= F.R) slot -= F.R;
        if (p0 + j == t) return fio + (size_t)stream * a.c + cc;  // the current token is not in the tail yet
        return tl + ((size_t)stream * F.R + slot) * a.c + cc;
      };
      region(F.m * fch, fz_l, [&](int qq) { return src(qq, 1); });
      region(F.m * fch, fx_l, [&](int qq) { return src(qq, 0); });
      if (F.bias_a)
        region(F.m * fW / 4, fb_l, [&](int qq) -> const void* {
          return F.bias_a + (size_t)(qq / (fW / 4)) * a.c + fr0 + 4 * (qq % (fW / 4));
        });
    }
    region(H * fch, fq_l, [&](int qq) -> const void* {
      return reinterpret_cast<const uint16_t*>(a.q) + ((size_t)qrow * H + qq / fch) * kC + fr0 + 8 * (qq % fch);
    });
    region(3 * fch, fa_l, [&](int qq) -> const void* {
      const int which = qq / fch, cc = fr0 + 8 * (qq % fch);
      return which == 0 ? reinterpret_cast<const uint16_t*>(F.x_new) + (size_t)b * a.c + cc
                        : fio + (size_t)(which - 1) * a.c + cc;
    });
  }

  if (tid == 0) s_restart = 0;
  // PG: page ids of the split's cache rows [r_begin, min(r_end, n_c))
  const int sh = a.pg.shift, p_first = SP ? 0 : r_begin >> sh;
  if constexpr (SP) {
    // the selected entries of rows [r_begin, min(r_end, n_c)): their cache
    // rows (paged: through the block table, a second round of loads)
    const int ce = r_end < nc32 ? r_end : nc32;
    const int32_t* ids = a.topk_idx + (size_t)qrow * a.k;
    for (int i0 = r_begin; i0 < ce; i0 += 256) {  // (a uniform loop)
      const int j = i0 + tid;
      if (j < ce) {
        const int32_t id = ids[j];
        int32_t row = -1;
        if (id >= 0 && id < a.E_cap) row = PG ? (int32_t)page_row(a.pg, b, id, a.E_cap) : id;
        s_pg[j - r_begin] = row;
      }
    }
  } else if constexpr (PG) {
    const int ce = r_end < nc32 ? r_end : nc32;
    if (r_begin < ce) {
      int np = ((ce - 1) >> sh) - p_first + 1;
      np = np < kPgSplit ? np : kPgSplit;  // (the rest: row_src reads the table)
      const int32_t* tb = a.pg.table + (size_t)b * (a.E_cap >> sh) + p_first;
      for (int i0 = 0; i0 < np; i0 += 256)  // (a uniform loop)
        if (i0 + tid < np) s_pg[i0 + tid] = tb[i0 + tid];
    }
  }
  __syncthreads();  // s_restart (and s_pg) ready

  auto spread4 = [](uint32_t x) { return (x & 1u) | ((x & 2u) << 7) | ((x & 4u) << 14) | ((x & 8u) << 21); };
  // source of the lane's row j of the split (branch-free); valid: j < r_end
  auto row_src = [&](int j) -> const uint16_t* {
    int wr = wbase + (j - nc32);
    wr = wr >= wcap ? wr - wcap : wr;
    size_t cr = (size_t)j;  // the cache row of entry j
    bool ok = true;         // SP: a selected id inside the cache
    if constexpr (SP) {
      int pi = j - r_begin;
      pi = pi < 0 ? 0 : (pi >= kPgSplit ? kPgSplit - 1 : pi);  // (rows that are not entries)
      const int32_t r = s_pg[pi];
      ok = r >= 0;
      cr = (size_t)(uint32_t)(ok ? r : 0);
    } else if constexpr (PG) {
      int pi = (j >> sh) - p_first;
      int32_t pg;
      if (pi >= kPgSplit && j < nc32) {
        // a page past the LDS table (splits of more than kPgSplit pages): its
        // id from the block table (the wait for it also waits for the DMAs
        // in flight)
        pg = a.pg.table[(size_t)b * (a.E_cap >> sh) + (j >> sh)];
      } else {
        pi = pi < 0 ? 0 : (pi >= kPgSplit ? kPgSplit - 1 : pi);  // (rows that are not entries)
        pg = s_pg[pi];
      }
      cr = ((size_t)(uint32_t)pg << sh) + (size_t)(j & ((1 << sh) - 1));
    }
    return j < r_end ? (j < nc32 ? (ok ? kv + cr * kC : pad_row) : win + (size_t)wr * kC) : pad_row;
  };
  auto set_valid = [&](int r0, int buf) {
    const int j = r0 + kRowsPerWave * w + (l & (kRowsPerWave - 1));
    bool okr = j < r_end;
    if constexpr (SP) {  // (an id outside the cache: a masked row)
      if (okr && j < nc32) okr = s_pg[j - r_begin] >= 0;
    }
    const uint64_t okb = __builtin_amdgcn_ballot_w64(okr);
    if (l == 0) {  // byte r % 4 of word r / 4: rows kRowsPerWave * w + i
      rvalid[buf][2 * w] = spread4((uint32_t)okb & 15u);
      rvalid[buf][2 * w + 1] = spread4((uint32_t)(okb >> 4) & 15u);
    }
  };
  auto issue_tile = [&](int r0, int buf) {
    dma_rows(row_src(r0 + kRowsPerWave * w + (l & (kRowsPerWave - 1))), buf);
    set_valid(r0, buf);
  };

  // the first kRing - 1 tiles (a pass recomputed after a jump of the
  // reference max)
  auto prologue = [&]() {
#pragma unroll
    for (int j = 0; j < kRing - 1; ++j)
      if (r_begin + j * kTN < r_end) issue_tile(r_begin + j * kTN, j);
  };
  // the speculative tile holds the right rows when every row of it that
  // the split uses is a cache entry; else it is fetched again
  if (spec && (r_end < r_begin + kTN ? r_end : r_begin + kTN) <= nc32) {
    set_valid(r_begin, 0);
  } else {
    __builtin_amdgcn_s_waitcnt(wait_vm(0));  // (the slot is written again)
    if (r_begin < r_end) issue_tile(r_begin, 0);
  }
  // every load and DMA so far (the query operands, the first tile, the
  // fold's inputs) has landed before the fold and the row loop; then the
  // next two tiles go out
  __builtin_amdgcn_s_waitcnt(0);
  __asm__ __volatile__("" ::"v"(qf[0]), "v"(qf[15]));
#pragma unroll
  for (int j = 1; j < kRing - 1; ++j)
    if (r_begin + j * kTN < r_end) issue_tile(r_begin + j * kTN, j);

  if (fW > 0) {
    lds_barrier();  // every wavefront's fold DMAs
    if (fold_now) {
      // thread (coordinate fc, source group fg of G = 256 / fW) folds
      // sources fg, fg + G, ... of its coordinate; the G partial states of
      // a coordinate merge across lanes (xor fW .. 32) and then across the
      // wavefronts.  (Reads: the lanes of one source row are consecutive
      // coordinates, adjacent groups adjacent rows.)
      const int fc = tid % fW, fg = tid / fW, G = 256 / fW;
      const uint16_t* zr = reinterpret_cast<const uint16_t*>(fz_l) + fc;
      const uint16_t* xr = reinterpret_cast<const uint16_t*>(fx_l) + fc;
      const float* br = reinterpret_cast<const float*>(fb_l) + fc;
      // all kFoldS sources' reads in flight together, branch-free
      const bool has_bias = F.bias_a != nullptr;  // (else the bias region is not loaded)
      float lgv[kFoldS], xvv[kFoldS];
      float mx = -INFINITY;
#pragma unroll
      for (int u = 0; u < kFoldS; ++u) {
        const int j = fg + G * u;
        const bool ok = j < F.m;
        const int e = (ok ? j : 0) * fW;
        const float zb = br[e];
        // (every read is made; an absent source adds -inf, which keeps the
        // reads out of conditional blocks)
        lgv[u] = (bf16_to_f32(zr[e]) + (has_bias ? zb : 0.f)) + (ok ? 0.f : -INFINITY);
        xvv[u] = bf16_to_f32(xr[e]);
        mx = fmaxf(mx, lgv[u]);
      }
      float l_ = 0.f, a_ = 0.f;
#pragma unroll
      for (int u = 0; u < kFoldS; ++u) {
        const float e_ = lgv[u] == -INFINITY ? 0.f : __expf(lgv[u] - mx);
        l_ += e_;
        a_ += e_ * xvv[u];
      }
      Soft st{mx, l_, a_};
#pragma unroll
      for (int k = 3; k < 6; ++k) {  // xor fW .. 32 (fW >= 8)
        const int msk = 1 << k;
        if (msk < fW) continue;
        const Soft o{__shfl_xor(st.mx, msk, 64), __shfl_xor(st.l, msk, 64), __shfl_xor(st.acc, msk, 64)};
        st = soft_merge_sel(st, o);
      }
      if (l < fW) s_fpart[w][fc] = st;
      lds_barrier();
      if (tid < fW) {
        Soft acc0 = s_fpart[0][tid];
#pragma unroll
        for (int g = 1; g < 4; ++g) acc0 = soft_merge_sel(acc0, s_fpart[g][tid]);
        const uint16_t vb = f32_to_bf16(acc0.acc / acc0.l);
        s_fnew[tid] = bf16_to_f32(vb);
        reinterpret_cast<uint16_t*>(F.kv_cache)[frow * kC + fr0 + tid] = vb;
        a.fold_new[(size_t)b * kC + fr0 + tid] = vb;
      }
      lds_barrier();
    }
    // this slice's share of q_h . entry and q_h . token: thread (head,
    // 8 coordinates), summed over the fch lanes of a head
    {
      const uint16_t* xq = reinterpret_cast<const uint16_t*>(fa_l);  // x_new slice
      const int ng = H * fch;
      for (int g0 = 0; g0 < ng; g0 += 256) {
        const int g = g0 + tid;
        float pn = 0.f, po = 0.f;
        if (g < ng) {
          const int hh = g / fch, c8 = 8 * (g % fch);
          float qv[8], xv[8];
          unpack16(*reinterpret_cast<const uint4*>(fq_l + 2 * (hh * fW + c8)), (const bf16*)nullptr, qv);
          unpack16(*reinterpret_cast<const uint4*>(xq + c8), (const bf16*)nullptr, xv);
#pragma unroll
          for (int i = 0; i < 8; ++i) po += qv[i] * xv[i];
          if (fold_now) {
#pragma unroll
            for (int i = 0; i < 8; ++i) pn += qv[i] * s_fnew[c8 + i];
          }
        }
#pragma unroll
        for (int k = 0; k < 3; ++k) {  // fch <= 8
          const int o = 1 << k;
          if (o >= fch) break;
          po += __shfl_xor(po, o, 64);
          pn += __shfl_xor(pn, o, 64);
        }
        if (g < ng && g % fch == 0) {
          // this slice's own slot: (q . new entry, q . token) shares
          float* fs = a.fold_s + 2 * (((size_t)b * H + g / fch) * kFoldSlots + split);
          *reinterpret_cast<float2*>(fs) = float2{fold_now ? pn : 0.f, po};
        }
      }
    }
    // the token's share of the rings (every step)
    if (tid < 3 * fch) {
      const int which = tid / fch, cc = fr0 + 8 * (tid % fch);
      const bool small = t < 0x7fffffff;  // 32-bit remainders
      const int ws = small ? (int)((uint32_t)t % (uint32_t)F.n_win) : (int)(t % F.n_win);
      const int ts = small ? (int)((uint32_t)t % (uint32_t)F.R) : (int)(t % F.R);
      uint16_t* dst = which == 0 ? reinterpret_cast<uint16_t*>(F.win_ring) + ((size_t)b * F.n_win + ws) * a.c + cc
                                 : reinterpret_cast<uint16_t*>(F.tail) + (((size_t)b * 2 + (which - 1)) * F.R + ts) * a.c + cc;
      *reinterpret_cast<uint4*>(dst) = s_fapp[tid];
    }
    if (split == 0 && tid == 0) a.fold_row[b] = fold_now ? cnt + 1 : 0;
    // the tile waits below count DMAs only
    __builtin_amdgcn_s_waitcnt(wait_vm(0));
  }

  // running softmax state of this wavefront's 16 heads: the reference max
  // per head (identical in the 4 lane groups), the sum per lane over its own
  // rows; accumulator: O^T[128 d x 64 heads] for the wavefront's quarter of
  // the coordinates (acc[4 dtl + hb]: d 128 w + 16 dtl .., heads 16 hb ..)
  f32x4_t acc[32];
#pragma unroll
  for (int dt = 0; dt < 32; ++dt) acc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_lane = 0.f;

  // per-lane LDS byte offsets of the score and value reads
  const Bases bs = lane_bases(li, lg);
  const int* s_base = bs.s;
  const int* t_base = bs.t;

  // Scores and softmax weights of the tile in slot sb: S^T[32 rows x 16
  // heads] = K . Q^T as two 16-row blocks, each summed in two halves (even /
  // odd k steps): four independent MFMA chains.  With WithPV, the previous
  // tile's O^T[d x 64 heads] += V^T[d x 32 rows] . P^T[32 rows x 64 heads]
  // (slot vb, operands pa) runs interleaved with them: two independent MFMA
  // streams and their LDS reads keep the one wavefront per SIMD busy while
  // either waits.  Returns this wavefront's P^T block (the rows permuted as
  // the B operand wants).
  auto score_tile = [&](auto with_pv, int sb, int vb, const bf16x8_t* pa) -> bf16x8_t {
    constexpr bool kPV = decltype(with_pv)::value;
    const char* T = tiles[sb];
    const char* V = tiles[vb];
    constexpr int kRB = kTN / 16;
    static_assert(kRB == 2, "one row pair per tile");
    f32x4_t s2[kRB][2];
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) s2[rb][0] = s2[rb][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 8; ++t) {
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const int ks = 2 * t + k2;
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb)
          s2[rb][ks & 1] = mfma32(lds8(T + s_base[ks & 3] + rb * 16 * kRowB + 256 * (ks >> 2)), qf[ks], s2[rb][ks & 1]);
      }
      if constexpr (kPV) {
        // each V^T block (two transposed reads) serves four MFMAs, so a
        // tile is transpose-read once per workgroup
        const char* v0 = V + t_base[t] + 256 * w;
        const bf16x8_t va = cat8(ld_tr(v0), ld_tr(v0 + 16 * kRowB));
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) acc[4 * t + hb] = mfma32(va, pa[hb], acc[4 * t + hb]);
      }
    }
    if constexpr (kPV) {
      // eight fragment reads ahead, then one read per MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 1);
#pragma unroll
      for (int i = 0; i < 40; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 24, 1);
    } else {
      // keep 12 fragment reads in flight ahead of the MFMAs (lgkmcnt counts 15)
      __builtin_amdgcn_sched_group_barrier(0x100, 12, 1);
#pragma unroll
      for (int i = 0; i < 16 * kRB - 12; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 12, 1);
    }
    f32x4_t sv[kRB];
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) sv[rb] = s2[rb][0] + s2[rb][1];
    // softmax weights against a fixed reference max per head; lane holds
    // rows 16rb + 4lg + i of head li.  The reference is the first tile's max
    // and stays put while tile maxima exceed it by at most kSlack (log2
    // units), so weights stay <= 2^kSlack and the accumulator is never
    // rescaled.  A larger jump raises the reference and asks for the split
    // to be recomputed from its first row (at most once: the second pass
    // starts from the largest max of the first).
    float x[kRB][4];
    float mx = -INFINITY;
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      const uint32_t fl = rvalid[sb][4 * rb + lg];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[rb][i] = ((fl >> (8 * i)) & 1u) ? sv[rb][i] * sc2 : -INFINITY;
        mx = fmaxf(mx, x[rb][i]);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const bool jump = m_run != -INFINITY && mx > m_run + kSlack;
    if (__builtin_amdgcn_ballot_w64(jump) != 0ull && l == 0) s_restart = 1;
    if (m_run == -INFINITY || jump) m_run = mx;  // no weight so far, or a pass to be redone
    bf16x4_t pb[kRB];
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = (x[rb][i] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(x[rb][i] - m_run);
        l_lane += p[i];
      }
      pb[rb] = bf16x4_t{(__bf16)p[0], (__bf16)p[1], (__bf16)p[2], (__bf16)p[3]};
    }
    return __builtin_shufflevector(pb[0], pb[1], 0, 1, 2, 3, 4, 5, 6, 7);
  };
  // the last tile's O^T += V^T . P^T alone
  auto pv_tile = [&](int vb, const bf16x8_t* pa) {
    const char* V = tiles[vb];
#pragma unroll
    for (int dtl = 0; dtl < 8; ++dtl) {
      const char* v0 = V + t_base[dtl] + 256 * w;
      const bf16x8_t va = cat8(ld_tr(v0), ld_tr(v0 + 16 * kRowB));
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) acc[4 * dtl + hb] = mfma32(va, pa[hb], acc[4 * dtl + hb]);
    }
    // two V^T blocks ahead, then one V^T block per four MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 2);
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 2);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 2);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 2);
  };
  // wait until at most `younger` of this wave's tiles issued after the one
  // needed next are still in flight (8 DMAs per tile)
  auto wait_tiles = [&](int younger) {
    if (younger >= 2) __builtin_amdgcn_s_waitcnt(wait_vm(2 * kRowsPerWave));
    else if (younger == 1) __builtin_amdgcn_s_waitcnt(wait_vm(kRowsPerWave));
    else __builtin_amdgcn_s_waitcnt(wait_vm(0));
  };

  // Ring of kRing tile slots, software-pipelined by one tile: iteration j
  // computes the scores of tile j+1 together with the P.V of tile j.  One
  // barrier per tile: before it each wave has published tile j's P^T block
  // and waited for its own DMAs of tile j+1; after it every wave may read
  // all P^T blocks of tile j and tile j+1, and every wave has finished the
  // P.V of tile j-1, whose slot then takes tile j+3 (tiles j+2, j+3 in
  // flight while j+1 is scored).  P^T alternates between two LDS buffers.
  static_assert(kRing == 4, "the waits below assume at most two younger tiles");
  for (;;) {
    const int nt = r_end > r_begin ? (r_end - r_begin + kTN - 1) / kTN : 0;
    if (nt > 0) {
      wait_tiles(nt - 1 < 2 ? nt - 1 : 2);  // tile 0 (tiles 1, 2 may be in flight)
      lds_barrier();
      // slot kRing - 1 is free now (the fold's staging is consumed)
      if (nt > 3) issue_tile(r_begin + 3 * kTN, 3);
      bf16x8_t pa[4];
      bf16x8_t pw = score_tile(std::false_type{}, 0, 0, pa);
      for (int j = 0;; ++j) {
        s_p[j & 1][w][l] = pw;
        // tiles issued so far: 0 .. min(max(j + 2, 3), nt - 1)
        const int hi = (j + 2 > 3 ? j + 2 : 3) < nt - 1 ? (j + 2 > 3 ? j + 2 : 3) : nt - 1;
        wait_tiles(hi - (j + 1) > 0 ? hi - (j + 1) : 0);
        lds_barrier();
        if (j >= 1 && j + 3 < nt) issue_tile(r_begin + (j + 3) * kTN, (j + 3) & (kRing - 1));
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) pa[hb] = s_p[j & 1][hb][l];
        if (j + 1 == nt) break;
        pw = score_tile(std::true_type{}, (j + 1) & (kRing - 1), j & (kRing - 1), pa);
      }
      pv_tile((nt - 1) & (kRing - 1), pa);
    }
    lds_barrier();
    const int again = s_restart;
    if (!again) break;
    // recompute the split against the raised reference maxima
    lds_barrier();
    if (tid == 0) s_restart = 0;
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) acc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    l_lane = 0.f;
    prologue();
  }

  // per-head sum over the four lane groups (this wavefront's 16 heads)
  float Lh = l_lane;
  Lh += __shfl_xor(Lh, 16, 64);
  Lh += __shfl_xor(Lh, 32, 64);
  const int h = h0 + li;

  // Output rows leave through LDS so that every store instruction writes one
  // contiguous 1 KB row.  The head owners publish their scales; lane (head
  // li of block hb) holds d = 128 w + 16 dtl + 4 lg + i of O^T and writes
  // them scaled and rounded to row 16 hb + li of the [64][520] bf16 staging
  // block (row stride 1040 B spreads the 8-byte writes over the banks);
  // then wavefront w copies the rows of its 16 heads, 16 bytes per lane.
  uint16_t* dst_row0;  // row of this wavefront's first head
  const size_t ostride = kC;
  {
    float f;  // output scale for this lane's head
    if (n_split == 1) {
      const float z2 = a.sink ? a.sink[h] * kLog2e : -INFINITY;
      const float M = fmaxf(m_run, z2);
      const float em = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - M);
      const float den = Lh * em + (z2 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(z2 - M));
      f = em / den;
      if (a.lse && lg == 0) a.lse[(size_t)qrow * H + h] = (M + log2f(den)) * kLn2;
      dst_row0 = reinterpret_cast<uint16_t*>(a.out) + ((size_t)qrow * H + h0) * kC;
    } else {
      // partial: (m, L) and O / L in bf16
      float* pml = reinterpret_cast<float*>(a.ws);
      uint16_t* po = reinterpret_cast<uint16_t*>(pml + (size_t)a.B * a.Tq * n_split * H * 2);
      const size_t slot = ((size_t)qrow * n_split + split) * H + h;
      if (lg == 0) {
        pml[2 * slot] = m_run;
        pml[2 * slot + 1] = Lh;
      }
      f = Lh > 0.f ? __builtin_amdgcn_rcpf(Lh) : 0.f;
      dst_row0 = po + (((size_t)qrow * n_split + split) * H + h0) * kC;
    }
    if (lg == 0) s_scale[16 * w + li] = f;
  }
  lds_barrier();
  constexpr int kOutLD = kC + 8;  // staging row stride (elements)
  uint16_t* stage = reinterpret_cast<uint16_t*>(tiles[0]);
#pragma unroll
  for (int hb = 0; hb < 4; ++hb) {
    const float f = s_scale[16 * hb + li];
#pragma unroll
    for (int dtl = 0; dtl < 8; ++dtl) {
      const f32x4_t v4 = acc[4 * dtl + hb];
      float x[4] = {v4[0] * f, v4[1] * f, v4[2] * f, v4[3] * f};
      // norm_rope: the rotary coordinates rotated back by the query position
      // (linear, so partials may be rotated before the merge)
      if (DEROT) rope_pairs<4>(x, 4, 128 * w + 16 * dtl + 4 * lg, kC, a.rope_dims, a.derot_freq, -t);
      ushort4 v;
      v.x = f32_to_bf16(x[0]);
      v.y = f32_to_bf16(x[1]);
      v.z = f32_to_bf16(x[2]);
      v.w = f32_to_bf16(x[3]);
      *reinterpret_cast<ushort4*>(stage + (16 * hb + li) * kOutLD + 128 * w + 16 * dtl + 4 * lg) = v;
    }
  }
  lds_barrier();
#pragma unroll
  for (int r = 0; r < 16; ++r)
    *reinterpret_cast<uint4*>(dst_row0 + r * ostride + 8 * l) =
        *reinterpret_cast<const uint4*>(stage + (16 * w + r) * kOutLD + 8 * l);
}

// grid (B*Tq, H), 256 threads: wavefront w merges splits w, w+4, ... of one
// head (lane = 8 coordinates), the four wavefronts add up through LDS.
constexpr int kMaxSplit = 64;
constexpr int kMergeU = kMaxSplit / 4;

__global__ __launch_bounds__(256) void attend_merge_kernel(AttendArgs a, int n_split) {
  __shared__ float s_o[4][64 * 8];
  __shared__ float s_den;
  const int qrow = blockIdx.x, h = blockIdx.y, tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int H = a.H;
  const float* pml = reinterpret_cast<const float*>(a.ws);
  const uint16_t* po = reinterpret_cast<const uint16_t*>(pml + (size_t)a.B * a.Tq * n_split * H * 2);
  const float z2 = a.sink ? a.sink[h] * kLog2e : -INFINITY;
  // fold_mode: the query's own token and the step's new entry (if any) as
  // two more rows, weights exp2(s_own - M) and exp2(s_new - M)
  const int b = qrow / a.Tq;
  const int frow = a.fold_mode ? a.fold_row[b] : 0;
  // the fold slices' shares of q . new entry and q . token, lane = slice,
  // summed in the same lane order on every run
  float2 fsv = float2{0.f, 0.f};
  if (a.fold_mode) {
    const int nf = (a.c + a.fold_cs - 1) / a.fold_cs;
    if (l < nf) fsv = *reinterpret_cast<const float2*>(a.fold_s + 2 * (((size_t)b * H + h) * kFoldSlots + l));
    fsv.x = wave_sum(fsv.x);
    fsv.y = wave_sum(fsv.y);
  }
  const float s_new = frow > 0 ? fsv.x * (a.scale * kLog2e) : -INFINITY;
  const float s_own = a.fold_mode ? fsv.y * (a.scale * kLog2e) : -INFINITY;
  // (fixed addresses: every load is issued at once)
  uint4 nrow = uint4{0, 0, 0, 0}, xrow = nrow;
  if (a.fold_mode) {
    nrow = *reinterpret_cast<const uint4*>(a.fold_new + (size_t)b * kC + 8 * l);
    xrow = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.fold.x_new) + (size_t)b * kC + 8 * l);
  }
  // this wavefront's splits' rows, then the statistics: every load is in
  // flight before the first wait
  uint4 raw[kMergeU];
#pragma unroll
  for (int u = 0; u < kMergeU; ++u) {
    const int s = w + 4 * u;
    raw[u] = uint4{0, 0, 0, 0};
    if (s < n_split) {
      const size_t slot = ((size_t)qrow * n_split + s) * H + h;
      raw[u] = *reinterpret_cast<const uint4*>(po + slot * kC + 8 * l);
    }
  }
  // lane s holds split s's statistics
  float ms = -INFINITY, Ls = 0.f;
  if (l < n_split) {
    const float2 v = *reinterpret_cast<const float2*>(pml + 2 * (((size_t)qrow * n_split + l) * H + h));
    ms = v.x;
    Ls = v.y;
  }
  const float M = fmaxf(fmaxf(fmaxf(wave_max(ms), z2), s_new), s_own);
  const float wgt = (ms == -INFINITY || Ls == 0.f) ? 0.f : __builtin_amdgcn_exp2f(ms - M) * Ls;
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < kMergeU; ++u) {
    const int s = w + 4 * u;  // < kMaxSplit = 64
    const float ws = __shfl(wgt, s, 64);
    if (s < n_split) {
      const uint32_t v[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o[2 * i] += ws * bf16_to_f32((uint16_t)(v[i] & 0xffff));
        o[2 * i + 1] += ws * bf16_to_f32((uint16_t)(v[i] >> 16));
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) s_o[w][8 * l + i] = o[i];
  const float w_new = frow > 0 ? __builtin_amdgcn_exp2f(s_new - M) : 0.f;
  const float w_own = a.fold_mode ? __builtin_amdgcn_exp2f(s_own - M) : 0.f;
  if (w == 0) {
    const float den = wave_sum(wgt) + (z2 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(z2 - M)) + w_new + w_own;
    if (l == 0) s_den = den;
  }
  __syncthreads();
  if (w != 0) return;
  if (a.fold_mode && l == 0 && h == 0 && frow > 0) a.fold.n_entries[b] = frow;  // publish the new entry count
  const float den = s_den;
  const float inv = __builtin_amdgcn_rcpf(den);
  const uint32_t nw[4] = {nrow.x, nrow.y, nrow.z, nrow.w}, xw[4] = {xrow.x, xrow.y, xrow.z, xrow.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float nv = bf16_to_f32((uint16_t)((nw[i >> 1] >> (16 * (i & 1))) & 0xffff));
    const float xv = bf16_to_f32((uint16_t)((xw[i >> 1] >> (16 * (i & 1))) & 0xffff));
    // (the new entry's row holds old data when no entry was completed)
    o[i] = (s_o[0][8 * l + i] + s_o[1][8 * l + i] + s_o[2][8 * l + i] + s_o[3][8 * l + i] +
            (frow > 0 ? w_new * nv : 0.f) + w_own * xv) *
           inv;
  }
  if (a.derot_freq) {  // norm_rope: the rotary pairs of the lane's 8 coordinates rotated back by t
    const int64_t t = a.q_pos ? a.q_pos[qrow] : a.q_pos0 + qrow % a.Tq;
    rope_pairs<8>(o, 8, 8 * l, kC, a.rope_dims, a.derot_freq, -t);
  }
  uint16_t* out = reinterpret_cast<uint16_t*>(a.out) + ((size_t)qrow * H + h) * kC + 8 * l;
  uint4 r;
  r.x = (uint32_t)f32_to_bf16(o[0]) | ((uint32_t)f32_to_bf16(o[1]) << 16);
  r.y = (uint32_t)f32_to_bf16(o[2]) | ((uint32_t)f32_to_bf16(o[3]) << 16);
  r.z = (uint32_t)f32_to_bf16(o[4]) | ((uint32_t)f32_to_bf16(o[5]) << 16);
  r.w = (uint32_t)f32_to_bf16(o[6]) | ((uint32_t)f32_to_bf16(o[7]) << 16);
  *reinterpret_cast<uint4*>(out) = r;
  if (a.lse && l == 0) a.lse[(size_t)qrow * H + h] = (M + log2f(den)) * kLn2;
}

bool attend_mfma_shape_ok(int H, int c) { return c == kC && H % kHW == 0; }

size_t attend_fold_ws_offset(int B, int Tq, int H, int c, int rows_max, int split_rows);
void attend_mfma_plan(int BT, int H, int rows_max, int split_rows, int* n_split, int* rows_per_split);

// HCA decode (one query per sequence, no overlap, bf16) with at least two
// row splits (the merge adds the new entry): the coordinates split into
// power-of-two slices of 8..64, one per split, every source token of a
// block handled by one thread of its slice.
bool attend_fuses_fold(AttendArgs& a, const FoldArgs& f) {
  a.fold_mode = 0;
  if (!a.dense || a.dtype != BF16 || f.dtype != BF16 || a.kv_fmt || f.kv_fmt ||
      !attend_mfma_shape_ok(a.H, a.c) ||
      a.Tq != 1 ||
      a.n_add != 0 || a.win_pos0 != nullptr || a.win_pos0_const != 0 || f.overlap || f.idx_dtype >= 0 ||
      f.B != a.B || f.c != a.c || f.n_win != a.W_cap || f.R < 2 * f.m)
    return false;
  int ns, rps;
  attend_mfma_plan(a.B * a.Tq, a.H, a.E_cap + a.n_win, a.split_rows, &ns, &rps);
  if (ns < 2) return false;
  int cs = 8;
  while (cs * ns < a.c) cs *= 2;
  // LDS: the slice's sources fill at most one ring slot, its query slice
  // the P^T buffer
  if (cs > 64 || a.c / cs > kFoldSlots || f.m > kFoldS * (256 / cs) || f.m * cs * 8 > kTN * kRowB || a.H * cs * 2 > 4 * 64 * 16)
    return false;
  const size_t off = attend_fold_ws_offset(a.B, a.Tq, a.H, a.c, a.E_cap + a.n_win, a.split_rows);
  char* base = reinterpret_cast<char*>(a.ws);
  a.fold_s = reinterpret_cast<float*>(base + off);
  const size_t off_row = off + ((size_t)a.B * a.H * kFoldSlots * 8 + 255) / 256 * 256;
  a.fold_row = reinterpret_cast<int32_t*>(base + off_row);
  a.fold_new = reinterpret_cast<uint16_t*>(base + off_row + ((size_t)a.B * 4 + 255) / 256 * 256);
  a.fold = f;
  a.fold_cs = cs;
  a.fold_mode = 1;
  return true;
}

// Row splits per (query, head group): about one workgroup per CU (256), each
// split a multiple of 16 rows, at most kMaxSplit splits; or split_rows rows
// each whatever the batch.
void attend_mfma_plan(int BT, int H, int rows_max, int split_rows, int* n_split, int* rows_per_split) {
  if (split_rows > 0) {
    *rows_per_split = split_rows;
    *n_split = (rows_max + split_rows - 1) / split_rows;
    return;
  }
  const int cols = BT * (H / kHW);
  int want = 256 / cols;
  if (want < 1) want = 1;
  if (want > kMaxSplit) want = kMaxSplit;
  int rps = (rows_max + want - 1) / want;
  rps = (rps + 15) / 16 * 16;
  *rows_per_split = rps;
  *n_split = (rows_max + rps - 1) / rps;
}

size_t attend_mfma_ws_bytes(int BT, int H, int rows_max, int split_rows) {
  int ns, rps;
  attend_mfma_plan(BT, H, rows_max, split_rows, &ns, &rps);
  if (ns <= 1) return 0;
  return (size_t)BT * ns * H * (2 * sizeof(float) + kC * sizeof(uint16_t));
}

hipError_t launch_attend_merge(const AttendArgs& a, int n_split, hipStream_t s);

// sparse rows on the 64-head kernel: for batches of many queries (the plan
// cuts no query's rows, so each selected row is gathered once per query and
// 64 heads), when a split's rows fit the LDS table.  Fewer queries (decode)
// go to the 16-head gather kernel, whose row splits fill the device.
bool attend_mfma_sparse_fits(const AttendArgs& a, int rows_max) {
  if (a.B * a.Tq * (a.H / kHW) < 256) return false;
  int ns, rps;
  attend_mfma_plan(a.B * a.Tq, a.H, rows_max, a.split_rows, &ns, &rps);
  return rps <= kPgSplit;
}

hipError_t launch_attend_mfma(const AttendArgs& a0, int rows_max, hipStream_t s) {
  int ns, rps;
  attend_mfma_plan(a0.B * a0.Tq, a0.H, rows_max, a0.split_rows, &ns, &rps);
  AttendArgs a = a0;
  a.fold_nsplit = 0;
  a.fold_rows = 0;
  if (a.fold_mode && a.split_rows == 0) {
    // the folding splits take kFoldRowsLess fewer rows (the same split count)
    const int nf = (a.c + a.fold_cs - 1) / a.fold_cs;
    if (nf < ns) {
      int ro = (rows_max + nf * kFoldRowsLess + ns - 1) / ns;
      ro = (ro + 15) / 16 * 16;
      const int rf = ro - kFoldRowsLess;
      if (rf >= 16 && (long long)nf * rf + (long long)(ns - nf) * ro >= rows_max) {
        a.fold_nsplit = nf;
        a.fold_rows = rf;
        rps = ro;
      }
    }
  }
  const int n_hg = a.H / kHW;
  const long long units = (long long)ns * a.B * a.Tq;       // (query, split) pairs
  const long long blocks = (units + 7) / 8 * 8 * n_hg;      // padded to whole XCD rounds
  const dim3 grid((unsigned)blocks), blk(256);
  // norm_rope: with row splits the merge rotates the output back (the
  // kernel's de-rotating form has a slower register allocation)
  const bool derot = a.derot_freq && ns == 1;
  if (!a.dense) {  // the sparse rows of a selection (prefill-shaped batches)
    if (a.pg.table && derot)
      CSA_LAUNCH("attend_sparse_mfma", (attend_mfma_kernel<1, 0, 1, 1>), grid, blk, 0, s, a, ns, rps);
    else if (a.pg.table)
      CSA_LAUNCH("attend_sparse_mfma", (attend_mfma_kernel<0, 0, 1, 1>), grid, blk, 0, s, a, ns, rps);
    else if (derot)
      CSA_LAUNCH("attend_sparse_mfma", (attend_mfma_kernel<1, 0, 0, 1>), grid, blk, 0, s, a, ns, rps);
    else
      CSA_LAUNCH("attend_sparse_mfma", (attend_mfma_kernel<0, 0, 0, 1>), grid, blk, 0, s, a, ns, rps);
  } else if (a.pg.table && derot)
    CSA_LAUNCH("attend_dense_mfma", (attend_mfma_kernel<1, 0, 1, 0>), grid, blk, 0, s, a, ns, rps);
  else if (a.pg.table && a.fold_mode)
    CSA_LAUNCH("attend_dense_mfma", (attend_mfma_kernel<0, 1, 1, 0>), grid, blk, 0, s, a, ns, rps);
  else if (a.pg.table)
    CSA_LAUNCH("attend_dense_mfma", (attend_mfma_kernel<0, 0, 1, 0>), grid, blk, 0, s, a, ns, rps);
  else if (derot)
    CSA_LAUNCH("attend_dense_mfma", (attend_mfma_kernel<1, 0, 0, 0>), grid, blk, 0, s, a, ns, rps);
  else if (a.fold_mode)
    CSA_LAUNCH("attend_dense_mfma", (attend_mfma_kernel<0, 1, 0, 0>), grid, blk, 0, s, a, ns, rps);
  else
    CSA_LAUNCH("attend_dense_mfma", (attend_mfma_kernel<0, 0, 0, 0>), grid, blk, 0, s, a, ns, rps);
  if (ns > 1) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_attend_merge(a, ns, s);
  }
  return hipGetLastError();
}

// Few splits and no fold: grid (B*Tq, H/4), wavefront w merges every split
// of head 4 y + w by itself (lane = 8 coordinates), so no workgroup
// exchange is needed.  The same combination as attend_merge_kernel.
constexpr int kMergeSmall = 16;
__global__ __launch_bounds__(256) void attend_merge_small_kernel(AttendArgs a, int n_split) {
  const int qrow = blockIdx.x, w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int h = blockIdx.y * 4 + w;
  const int H = a.H;
  const float* pml = reinterpret_cast<const float*>(a.ws);
  const uint16_t* po = reinterpret_cast<const uint16_t*>(pml + (size_t)a.B * a.Tq * n_split * H * 2);
  // every split's row, then the statistics: all loads in flight before the
  // first wait
  uint4 raw[kMergeSmall];
#pragma unroll
  for (int u = 0; u < kMergeSmall; ++u) {
    raw[u] = uint4{0, 0, 0, 0};
    if (u < n_split) raw[u] = *reinterpret_cast<const uint4*>(po + (((size_t)qrow * n_split + u) * H + h) * kC + 8 * l);
  }
  float ms = -INFINITY, Ls = 0.f;
  if (l < n_split) {
    const float2 v = *reinterpret_cast<const float2*>(pml + 2 * (((size_t)qrow * n_split + l) * H + h));
    ms = v.x;
    Ls = v.y;
  }
  const float z2 = a.sink ? a.sink[h] * kLog2e : -INFINITY;
  const float M = fmaxf(wave_max(ms), z2);
  const float wgt = (ms == -INFINITY || Ls == 0.f) ? 0.f : __builtin_amdgcn_exp2f(ms - M) * Ls;
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < kMergeSmall; ++u) {
    const float ws = __shfl(wgt, u, 64);
    if (u < n_split) {
      const uint32_t v[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o[2 * i] += ws * bf16_to_f32((uint16_t)(v[i] & 0xffff));
        o[2 * i + 1] += ws * bf16_to_f32((uint16_t)(v[i] >> 16));
      }
    }
  }
  const float den = wave_sum(wgt) + (z2 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(z2 - M));
  const float inv = __builtin_amdgcn_rcpf(den);
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] *= inv;
  if (a.derot_freq) {  // norm_rope: the rotary pairs of the lane's 8 coordinates rotated back by t
    const int64_t t = a.q_pos ? a.q_pos[qrow] : a.q_pos0 + qrow % a.Tq;
    rope_pairs<8>(o, 8, 8 * l, kC, a.rope_dims, a.derot_freq, -t);
  }
  uint16_t* out = reinterpret_cast<uint16_t*>(a.out) + ((size_t)qrow * H + h) * kC + 8 * l;
  uint4 r;
  r.x = (uint32_t)f32_to_bf16(o[0]) | ((uint32_t)f32_to_bf16(o[1]) << 16);
  r.y = (uint32_t)f32_to_bf16(o[2]) | ((uint32_t)f32_to_bf16(o[3]) << 16);
  r.z = (uint32_t)f32_to_bf16(o[4]) | ((uint32_t)f32_to_bf16(o[5]) << 16);
  r.w = (uint32_t)f32_to_bf16(o[6]) | ((uint32_t)f32_to_bf16(o[7]) << 16);
  *reinterpret_cast<uint4*>(out) = r;
  if (a.lse && l == 0) a.lse[(size_t)qrow * H + h] = (M + log2f(den)) * kLn2;
}

hipError_t launch_attend_merge(const AttendArgs& a, int n_split, hipStream_t s) {
  if (n_split > kMaxSplit) return hipErrorInvalidValue;
  if (!a.fold_mode && n_split <= kMergeSmall && a.H % 4 == 0) {
    CSA_LAUNCH("attend_merge", attend_merge_small_kernel, dim3(a.B * a.Tq, a.H / 4), dim3(256), 0, s, a, n_split);
    return hipGetLastError();
  }
  CSA_LAUNCH("attend_merge", attend_merge_kernel, dim3(a.B * a.Tq, a.H), dim3(256), 0, s, a, n_split);
  return hipGetLastError();
}

}  // namespace csa
