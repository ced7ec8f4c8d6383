// Grouped SwiGLU expert FFN over variable-length row segments.
//
// Role: the grouped GEMM that the paper review ("Improving MoE Compute
// Efficiency by Composing Weight and Data Sparsity", section 3
// "implementation") calls on the truncated, expert-sorted slot list, so the
// null slots never reach it. The expert is a per-token FFN (quant67 MoE
// primer, section 2) in SwiGLU form:
//     h = silu(W_gate a) * (W_up a),   out = W_down h,   silu(z) = z / (1 + e^-z)
//
// bf16 path, MI355X design:
//  * v_mfma_f32_32x32x16_bf16 with float32 accumulation. The MFMA "A" operand
//    is the weight tile and "B" the activation tile, so each lane ends up with
//    four consecutive output columns of one row (8-byte bf16 / 16-byte fp32
//    stores). h is stored in bf16 because the down projection's MFMA reads
//    bf16; the expert output stays float32 so that the combine rounds the
//    layer output only once.
//  * Workgroup tile BM rows x BN weight rows x 64 K (default 128 x 256 on eight
//    wavefronts of 64 x 64). For the gate/up pass the BN weight rows are BN/2 gate
//    + BN/2 up rows of the same output columns, so a lane holds gate and up values
//    of the same (row, column) and applies SwiGLU in registers; h is written once.
//  * K tiles stream through S LDS stages filled by buffer->LDS loads
//    (buffer_load_dwordx4 ... lds): no staging registers, S-1 tiles in flight
//    while one is multiplied, and the wait before each barrier counts only this
//    wavefront's loads issued after the tile about to be read. The loads of the
//    next tile are spread between the MFMA steps: the CU's address unit takes one
//    1 KB load at a time, so issuing them all after the barrier stalled every
//    wavefront. LDS rows are 128 bytes with 16-byte chunks XOR-swizzled by
//    (row / 2) mod 8, so the 16 rows one pass of a fragment read touches fall in
//    distinct banks of the 64; the swizzle is applied on the global side of each
//    load. A stage's fragment reads are all issued before its MFMAs, each MFMA
//    step waiting only for its own reads.
//  * Persistent grid. Each workgroup builds the tile table from the device
//    offsets (no host round trip for R), and tiles are ordered
//    (expert, column tile, row tile) for a grouped problem and (row tile, column
//    tile) for a dense one; each problem's list is cut into 8 contiguous ranges, one
//    per XCD (workgroups are dispatched round-robin over the 8 XCDs). The tiles an
//    XCD runs at once then share one expert's weight panel (grouped: the weights are
//    the larger operand of a segment) or a few activation row panels (dense: the
//    activations are read about once instead of once per column tile).
//  * When a range's last round has fewer tiles than the range has workgroups,
//    those tiles are split by output columns into 2 or 4 sub-tiles, so every
//    workgroup streams about the same weight bytes. Rows past the segment or
//    outside the sub-tile are read one row past their buffer's end (zero, no
//    memory traffic). Each workgroup fetches the next item's row indices while it
//    multiplies the current item, and issues the next item's first stages before
//    it stores the current item's outputs.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

// Groups of one launch's two problems together: the backward pairs two grouped
// problems of up to MOE_MAX_EXPERTS (255) groups each (gate and up), or 255 routed
// groups and up to 32 chunks of the shared expert. The tile table lives in LDS next
// to the stages (7 x 513 ints, 14 KB).
constexpr int kMaxGroups = 512;

// kSwiGLU: h = silu(a b0^T) * (a b1^T), a and both weights bf16, h stored as IEEE half.
// kPlain:  out = a b0^T, a and b0 bf16, float32 out.
// kDown16: out = h b0^T with h IEEE half (the layer's intermediate) and b0 bf16, each
//          weight fragment widened to half in registers (exact for |w| >= 2^-17) so the
//          MFMA runs in half precision; float32 out.
// kDownComb: kDown16 for the shared expert of the layer, whose epilogue adds the
//          token's weighted routed expert outputs (the combine) and stores bf16 y
//          (256 x 256 tiles only).
// kPlainKM: kPlain with K-major weights (GemmProblem::b_kmajor; 256 x 256 tiles only): the
//          weight tile is staged in LDS as [K][weight rows] and its MFMA fragments are
//          read with the transposing LDS load (ds_read_b64_tr_b16), so no transposed copy
//          of the weights is written.
// kPlainKM2: kPlainKM whose activation operand is K-major too (GemmProblem::a_kmajor, the
//          weight-gradient form: K = rows of both source matrices), read the same way.
// kSwiGLUKeep: kSwiGLU for the backward's recompute (256 x 256 tiles only): the epilogue
//          stores g and u (IEEE half, keep_g / keep_u) and h = silu(g) u as bf16 (from the
//          float32 g and u).
enum { kSwiGLU = 0, kPlain = 1, kDown16 = 2, kDownComb = 3, kPlainKM = 4, kPlainKM2 = 5, kSwiGLUKeep = 6 };

// One 32x32x16 MFMA step: the weight fragment w (bf16 bits) and the activation
// fragment a (bf16 bits, or half bits for kDown16).
template <int MODE>
__device__ __forceinline__ f32x16_t mfma32(bf16x8_t w, bf16x8_t a, f32x16_t c) {
  if constexpr (MODE == kDown16 || MODE == kDownComb)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(bf16x8_to_f16x8(w), __builtin_bit_cast(f16x8_t, a), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(w, a, c, 0, 0, 0);
}

// Element offset of (row, 16-byte chunk) in a [rows][BK] bf16 LDS tile. The LDS
// has 64 four-byte banks, and a 16-byte read serves 16 lanes per pass, here 16
// consecutive rows at one logical chunk. 128-byte rows (BK = 64) XOR the chunk with
// (row / 2) % 8: an even and an odd row cover the two 128-byte halves of the banks,
// and the 8 even (8 odd) rows take 8 distinct chunks. 64-byte rows (BK = 32) XOR
// with (row / 4) % 4 for the same reason. (XOR with row % 8 leaves two-way
// conflicts: measured 120 against 181 bytes per clock per CU.)
template <int BK>
__device__ __forceinline__ int lds_off(int row, int chunk) {
  if constexpr (BK == 64) return row * 64 + ((chunk ^ ((row >> 1) & 7)) << 3);
  else return row * 32 + ((chunk ^ ((row >> 2) & 3)) << 3);
}

// Scheduling pins for one multiplied K tile after its LDS reads: for each of the KS
// MFMA steps, the tile loads issued there (part ks of J, none when NJ is 0), then the
// step's NM MFMAs.
constexpr int loads_in_part(int nj, int ks_count, int ks) {
  int c = 0;
  for (int j = 0; j < nj; ++j) c += j * ks_count / nj == ks;
  return c;
}
template <int NJ, int KS, int NM, int KSI = 0>
__device__ __forceinline__ void sched_steps() {
  if constexpr (KSI < KS) {
    constexpr int nl = loads_in_part(NJ, KS, KSI);
    if constexpr (nl > 0) __builtin_amdgcn_sched_group_barrier(0x010, nl, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
    sched_steps<NJ, KS, NM, KSI + 1>();
  }
}

struct TileTable {
  int start[kMaxGroups + 1];
  int len[kMaxGroups + 1];
  int mt[kMaxGroups + 1];
  int nt[kMaxGroups + 1];
  int prefix[kMaxGroups + 1];
  int kofs[kMaxGroups + 1];  // K range of each group (k_offsets problems; else 0, k_dim)
  int klen[kMaxGroups + 1];
};

// Table of the tiles of problem 0's groups followed by
// problem 1's single dense group. Segment e of a grouped problem is [a, b) with
// a = clamp(offsets[e], 0, max_rows), b = clamp(offsets[e+1], a, max_rows):
// always inside the buffers, exactly the requested segment for valid offsets.
__device__ void build_tile_table(TileTable& tt, const GemmProblem& p0, const GemmProblem& p1,
                                 int oc, int bm) {
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    const int G0 = p0.groups, G = p0.groups + p1.groups;
    constexpr int kPer = (kMaxGroups + kWave - 1) / kWave;
    int cnt[kPer], local = 0;
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int e = lane * kPer + q;
      int s = 0, l = 0, nt = 0, ko = 0, kl = 0;
      if (e < G) {
        const GemmProblem pr = e < G0 ? p0 : p1;
        const int ge = e < G0 ? e : e - G0;
        kl = pr.k_dim;
        if (pr.k_offsets) {  // clamped to [0, k_dim] as the segments are to [0, max_rows]
          ko = min(max(pr.k_offsets[ge], 0), pr.k_dim);
          kl = min(max(pr.k_offsets[ge + 1], ko), pr.k_dim) - ko;
        }
        if (pr.rows_per_group > 0) {
          const int64_t a = min<int64_t>((int64_t)ge * pr.rows_per_group, pr.max_rows);
          s = (int)a;
          l = (int)(min<int64_t>(a + pr.rows_per_group, pr.max_rows) - a);
        } else if (pr.offsets) {
          int64_t a = pr.offsets[ge], b = pr.offsets[ge + 1];
          a = min<int64_t>(max<int64_t>(a, 0), pr.max_rows);
          b = min<int64_t>(max<int64_t>(b, a), pr.max_rows);
          s = (int)a;
          l = (int)(b - a);
        } else {
          l = (int)pr.max_rows;
        }
        nt = (pr.n_out + oc - 1) / oc;
      }
      const int m = (l + bm - 1) / bm;
      if (e <= kMaxGroups) {
        tt.start[e] = s;
        tt.len[e] = l;
        tt.mt[e] = m;
        tt.nt[e] = nt;
        tt.kofs[e] = ko;
        tt.klen[e] = kl;
      }
      cnt[q] = m * nt;
      local += cnt[q];
    }
    int incl = local;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int v = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += v;
    }
    int run = incl - local;
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int e = lane * kPer + q;
      if (e <= kMaxGroups) tt.prefix[e] = run;
      run += cnt[q];
    }
    if (lane == kWave - 1) tt.prefix[kMaxGroups] = incl;
  }
  __syncthreads();
}

// Row tile and column tile of tile `local` of a group with mt row tiles and nt
// column tiles. A dense problem (one group of max_rows rows) runs row-major, a
// grouped one column-major (all row tiles of one column panel in a row).
__device__ __forceinline__ void tile_of(const GemmProblem& pr, int local, int mt, int nt,
                                        int& mtile, int& ntile) {
  if (pr.groups == 1 && !pr.offsets && pr.rows_per_group <= 0) {
    mtile = local / nt;
    ntile = local - mtile * nt;
  } else {
    ntile = local / mt;
    mtile = local - ntile * mt;
  }
}

// Workgroups of a tile shape that fit one CU's 160 KB of LDS (stages + tile table);
// the register budget per wavefront follows from it.
constexpr int gemm_groups_per_cu(int bm, int bn, int s, int bk) {
  return (int)((160 * 1024) / ((size_t)s * (bm + bn) * bk * 2 + sizeof(TileTable)));
}

// MODE kSwiGLU writes h as bf16 (the next MFMA's input); kPlain writes float32.
// ROLE only names the launch in profiles (the code is identical): 0 standalone
// grouped, 1 standalone single segment, 2 the layer's routed + shared launch, 3 the
// layer backward's launches.
//
// Tile BM rows x BN weight rows x BK K on WM x WN wavefronts; each wavefront owns
// (BM/WM) x (BN/WN) outputs as 32x32 MFMA blocks. K tiles stream through S LDS
// stages filled by buffer->LDS loads: no staging registers, S-1 stages in flight
// while one is multiplied. One wavefront load instruction fills 1 KB of LDS: 8 rows
// of 128 bytes (BK = 64) or 16 rows of 64 bytes (BK = 32), lane l writing physical
// chunk l % CPR of row l / CPR; it fetches the logical chunk that lds_off() places
// there, which realises the XOR swizzle that keeps the MFMA fragment reads free of
// bank conflicts. (The buffer form, not global_load_lds: the compiler counts the
// global form as a possible LDS-side event and then waits for every LDS read at
// once.)
template <int MODE, int ROLE, int BM, int BN, int WM, int WN, int S, int BK>
__global__ void __launch_bounds__(64 * WM * WN)
__attribute__((amdgpu_waves_per_eu(WM * WN / 4 * gemm_groups_per_cu(BM, BN, S, BK),
                                   WM * WN / 4 * gemm_groups_per_cu(BM, BN, S, BK))))
grouped_gemm_bf16_kernel(GemmProblem p0, GemmProblem p1) {
  static_assert(BK == 32 || BK == 64, "K tile of 64- or 128-byte rows");
  constexpr int NW = WM * WN;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int OC = MODE == kSwiGLU ? BN / 2 : BN;  // output columns per tile
  constexpr int CPR = BK / 8;                        // 16-byte chunks per tile row
  constexpr int RPI = kWave / CPR;                   // tile rows filled by one load instruction
  constexpr int J = (BM + BN) / (RPI * NW);          // load instructions per stage per wavefront
  constexpr int JA = BM / (RPI * NW);                // of which fill A rows
  constexpr int STAGE = (BM + BN) * BK;              // elements per stage
  static_assert(BM % (RPI * NW) == 0 && BN % (RPI * NW) == 0, "tile rows must split over the wavefronts");
  static_assert(MODE != kSwiGLU || FN % 2 == 0, "gate/up tiles come in pairs");
  static_assert(S >= 2 && S <= 6 && J * (S - 2) + JA < 64, "loads in flight must fit the vmcnt counter");
  __shared__ TileTable tt;
  extern __shared__ __attribute__((aligned(16))) bf16_t smem[];  // [S][BM + BN][BK]
  build_tile_table(tt, p0, p1, OC, BM);
  const int G0 = p0.groups, G = p0.groups + p1.groups;
  const int total = tt.prefix[kMaxGroups];

  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave % WM, wn = wave / WM;
  const int half = lane >> 5, l32 = lane & 31;
  // this lane's load: row RPI (wave + NW j) + lane / CPR of the stage, physical chunk
  // lane % CPR, so logical chunk lc (the swizzle of lds_off, which depends only on
  // the row's offset within the instruction's RPI rows)
  // (the instruction's first row is RPI (wave + NW j): a multiple of 16 for BK = 32,
  // and for BK = 64 a multiple of 8 whose half-row parity is that of wave, NW being even)
  static_assert(BK == 32 || NW % 2 == 0, "the load swizzle assumes an even wavefront count");
  const int lrow = lane / CPR;
  const int lc = (lane % CPR) ^ (BK == 64 ? (((wave & 1) << 2) | (lrow >> 1)) : (lrow >> 2) & 3);

  // XCD-contiguous tile ranges: each XCD takes an eighth of problem 1's tiles
  // followed by an eighth of problem 0's, so a second problem (the dense shared
  // expert, whose tiles are long MFMA chains) is spread over every XCD instead of
  // filling the last ones. When a range's last round would leave workgroups idle,
  // its tiles (problem 0's last) are split by output columns into 2 or 4 sub-tiles,
  // so that every workgroup of the range streams about the same number of weight bytes.
  const int P = gridDim.x;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int Bx = P >> 3;
  const int T0 = tt.prefix[G0], T1 = total - T0;
  const int b0 = (int)((int64_t)xcd * T0 / 8), n0 = (int)((int64_t)(xcd + 1) * T0 / 8) - b0;
  const int b1 = T0 + (int)((int64_t)xcd * T1 / 8), n1 = T0 + (int)((int64_t)(xcd + 1) * T1 / 8) - b1;
  const int nx = n0 + n1;
  const int full = nx / Bx * Bx, rem = nx - full;
  const int split = rem == 0 ? 1 : (WN >= 4 && 4 * rem <= Bx) ? 4 : (WN >= 2 && 2 * rem <= Bx) ? 2 : 1;
  const int items = full + rem * split;

  // One work item: where its operands come from and where its outputs go. The
  // operands are read through buffer resources (the activation matrix; this group's
  // gate or up weight matrix) at 32-bit byte offsets, one row start per load. Rows
  // that feed nothing stored (past the segment, outside a sub-tile's columns) point
  // one row past the resource's end, where reads return zero without a memory access,
  // so every wavefront issues the same J loads per K tile.
  struct Tile {
    bool second, wact;
    int ge, Kdim, nk, m0, rows_valid, col0;
    __amdgpu_buffer_rsrc_t ra, rb0, rb1;
    uint32_t a_end, b_end;  // one past each resource (reads there return zero)
    uint32_t off[J];
  };
  // Locates work item it (group, row tile, column tile, sub-tile columns), decides
  // which load instructions fetch something used (A rows before rows_valid, weight
  // rows of the sub-tile's columns; wave-uniform and the same for every K tile, so
  // each stage of the item holds jn of this wavefront's loads) and sets each load's
  // row source, always a valid row: rows past the segment and columns past n_out
  // only feed outputs that are never stored.
  struct Where {
    bool second;
    int ge, Kdim, kofs, nk, m0, rows_valid, col0, ocp;
  };
  auto locate = [&](int it, Where& w) {
    int i = it, part = 0, parts = 1;
    if (it >= full) {
      i = full + (it - full) / split;
      part = (it - full) % split;
      parts = split;
    }
    const int L = i < n1 ? b1 + i : b0 + (i - n1);
    int lo = 0, hi = G;  // prefix[lo] <= L < prefix[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (tt.prefix[mid] <= L) lo = mid; else hi = mid;
    }
    const int e = lo;
    w.second = e >= G0;
    const GemmProblem pr = w.second ? p1 : p0;
    w.ge = w.second ? e - G0 : e;
    w.Kdim = tt.klen[e];
    w.kofs = tt.kofs[e];
    w.nk = (w.Kdim + BK - 1) / BK;
    const int local = L - tt.prefix[e];
    int mtile, ntile;
    tile_of(pr, local, tt.mt[e], tt.nt[e], mtile, ntile);
    w.m0 = __builtin_amdgcn_readfirstlane(tt.start[e] + mtile * BM);
    w.rows_valid = __builtin_amdgcn_readfirstlane(min(BM, tt.start[e] + tt.len[e] - w.m0));
    w.ocp = OC / parts;  // output columns of this item
    w.col0 = __builtin_amdgcn_readfirstlane(ntile * OC + part * w.ocp);
  };
  // First half of an item's set-up: where it is and the row indices of its A loads
  // (global loads of a_rows for a gathered problem). Issued one item ahead, so their
  // latency passes during the current item's K loop.
  struct Pre {
    Where w;
    int64_t arow[JA > 0 ? JA : 1];
  };
  auto fetch = [&](int it, Pre& q) {
    locate(it, q.w);
    const GemmProblem pr = q.w.second ? p1 : p0;
#pragma unroll
    for (int j = 0; j < JA; ++j) {
      const int r = RPI * (wave + NW * j) + lrow;
      q.arow[j] = q.w.m0 + (r < q.w.rows_valid ? r : 0);
    }
    if (pr.a_rows) {
#pragma unroll
      for (int j = 0; j < JA; ++j) q.arow[j] = pr.a_rows[q.arow[j]];
    }
  };
  // a_rows loads fetch() leaves in flight (wave-uniform)
  auto fetch_loads = [&](const Pre& q) { return (q.w.second ? p1 : p0).a_rows ? JA : 0; };
  auto setup = [&](const Pre& q, Tile& t) {
    const Where& w = q.w;
    t.second = w.second;
    t.ge = w.ge;
    t.Kdim = w.Kdim;
    t.nk = w.nk;
    t.m0 = w.m0;
    t.rows_valid = w.rows_valid;
    t.col0 = w.col0;
    const int ocp = w.ocp, parts = OC / ocp;
    const GemmProblem pr = t.second ? p1 : p0;
    const int Nout = pr.n_out;
    // wavefronts whose rows or columns all fall outside skip the MFMAs and the stores
    t.wact = __builtin_amdgcn_readfirstlane(wn < WN / parts && wm * TM < t.rows_valid);
    int64_t arow[JA > 0 ? JA : 1];
#pragma unroll
    for (int j = 0; j < JA; ++j)
      arow[j] = pr.a_rows ? min<int64_t>(max<int64_t>(q.arow[j], 0), pr.a_nrows - 1) : q.arow[j];
    const int64_t lda = pr.lda ? pr.lda : pr.k_dim, ldb = pr.ldb ? pr.ldb : pr.k_dim;
    const uint32_t a_rb = (uint32_t)lda * 2, b_rb = (uint32_t)ldb * 2;  // row strides, bytes
    // b0/b1: this group's matrix, or for k_offsets problems the one shared matrix,
    // entered at the group's first K column
    const int64_t wofs = pr.k_offsets ? (int64_t)w.kofs : (int64_t)t.ge * Nout * ldb;
    // gathered rows address the whole activation matrix ((rows + 1) x row bytes at
    // most 4 GB, checked on the host); a contiguous segment's resource covers just
    // the item's valid rows (for rows_per_group problems rows of the shared a)
    const int64_t abase = pr.a_rows ? 0 : t.m0 - (pr.rows_per_group ? (int64_t)t.ge * pr.rows_per_group : 0);
    const uint32_t a_end = (uint32_t)((pr.a_rows ? pr.a_nrows : t.rows_valid) * a_rb);
    const uint32_t b_end = (uint32_t)Nout * b_rb;
    t.a_end = a_end;
    t.b_end = b_end;
    t.ra = buffer_rsrc(pr.a + abase * lda + w.kofs, a_end);
    t.rb0 = buffer_rsrc(pr.b0 + wofs, b_end);
    t.rb1 = buffer_rsrc(MODE == kSwiGLU ? pr.b1 + wofs : pr.b0 + wofs, b_end);
#pragma unroll
    for (int j = 0; j < JA; ++j) {
      const int r = RPI * (wave + NW * j) + lrow;
      t.off[j] = r >= t.rows_valid ? a_end : pr.a_rows ? (uint32_t)arow[j] * a_rb : (uint32_t)r * a_rb;
    }
#pragma unroll
    for (int j = JA; j < J; ++j) {
      const int r = RPI * (wave + NW * j) + lrow - BM;
      const int c = MODE == kSwiGLU ? r % OC : r;  // output column within the tile
      const int n = t.col0 + c;
      t.off[j] = c < ocp && n < Nout ? (uint32_t)n * b_rb : b_end;
    }
  };
  // K tile kt of item t into stage st; with q >= 0 only the loads of part q of
  // BK / 16 (spread over the MFMA steps of the tile being multiplied). Chunks past
  // k_dim (last tile only) read column 0; they are zeroed in LDS before the MFMAs
  // read the stage. Past the item's last K tile every load reads past its resource's
  // end (zero, no memory access) into a stage that nothing reads before it is
  // refilled: the K loop body stays one straight instruction sequence.
  auto issue = [&](const Tile& t, int kt, int st, int q) {
    const bool past = kt >= t.nk;
    const int k = kt * BK + lc * 8;
    const uint32_t kb = (uint32_t)(k < t.Kdim ? k : 0) * 2;
    bf16_t* stage = smem + st * STAGE;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      if (q >= 0 && j * (BK / 16) / J != q) continue;
      // which resource: A rows, then gate (or plain) weight rows, then up rows
      const bool up = MODE == kSwiGLU && j >= JA && RPI * (wave + NW * j) - BM >= OC;
      const uint32_t end = j < JA ? t.a_end : t.b_end;
      buffer_load_lds16(j < JA ? t.ra : up ? t.rb1 : t.rb0, past ? end : t.off[j] + kb,
                        stage + RPI * (wave + NW * j) * BK);
    }
  };
  // the first S-1 K tiles of an item, into stages 0 .. S-2
  auto prologue = [&](const Tile& t) {
#pragma unroll
    for (int s = 0; s < S - 1; ++s)
      if (s < t.nk) issue(t, s, s, -1);
  };

  Tile cur;
  Pre pre;
  if (slot < items) {
    fetch(slot, pre);
    setup(pre, cur);
    prologue(cur);
  }
  for (int it = slot; it < items; it += Bx) {
    // the next item's row indices, behind this item's first S-1 K tiles
    const bool more = it + Bx < items;
    if (more) fetch(it + Bx, pre);
    const int na = more ? fetch_loads(pre) : 0;
    f32x16_t acc[FN][FM];
#pragma unroll
    for (int f = 0; f < FN; ++f)
#pragma unroll
      for (int g = 0; g < FM; ++g) acc[f][g] = f32x16_t{};

    // One K tile from stage st in four 16-wide steps; the fragments of step ks+1
    // are read while step ks multiplies.
    // With ISS, K tile nt's loads are issued between the MFMA steps (part ks before
    // step ks's MFMAs): the CU's address unit takes each 1 KB load in turn, so loads
    // issued by every wavefront at once after the barrier would hold up all MFMAs.
    auto compute = [&](auto iss, int st, int nt) {
      constexpr bool ISS = decltype(iss)::value;
      const bf16_t* As = smem + st * STAGE;
      const bf16_t* Bs = As + BM * BK;
      auto frags = [&](int ks, bf16x8_t* w, bf16x8_t* a) {
        const int ch = ks * 2 + half;
#pragma unroll
        for (int f = 0; f < FN; ++f) {
          int brow;
          if (MODE == kSwiGLU)
            brow = (f < FN / 2 ? 0 : BN / 2) + wn * (TN / 2) + (f % (FN / 2)) * 32 + l32;
          else
            brow = wn * TN + f * 32 + l32;
          w[f] = *reinterpret_cast<const bf16x8_t*>(&Bs[lds_off<BK>(brow, ch)]);
        }
#pragma unroll
        for (int g = 0; g < FM; ++g)
          a[g] = *reinterpret_cast<const bf16x8_t*>(&As[lds_off<BK>(wm * TM + g * 32 + l32, ch)]);
      };
      constexpr int KS = BK / 16;
      if constexpr ((FN + FM) * KS * 4 <= 64) {
        // All of the stage's fragment reads are issued first (64 VGPRs at most), so
        // each 16-wide step's MFMAs wait only for their own reads (LDS reads return
        // in order) while the later ones are still in flight.
        bf16x8_t wa[KS][FN], aa[KS][FM];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) frags(ks, wa[ks], aa[ks]);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          if constexpr (ISS) issue(cur, nt, nt % S, ks);
#pragma unroll
          for (int f = 0; f < FN; ++f)
#pragma unroll
            for (int g = 0; g < FM; ++g)
              acc[f][g] = mfma32<MODE>(wa[ks][f], aa[ks][g], acc[f][g]);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, (FN + FM) * KS, 0);  // LDS reads
        sched_steps<ISS ? J : 0, KS, FN * FM>();  // then per step: its loads, its MFMAs
      } else {
        // larger wavefront tiles: fragments of step ks + 1 are read while step ks multiplies
        bf16x8_t wf[2][FN], af[2][FM];
        frags(0, wf[0], af[0]);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int cb = ks & 1;
          if (ks + 1 < KS) frags(ks + 1, wf[cb ^ 1], af[cb ^ 1]);
          if constexpr (ISS) issue(cur, nt, nt % S, ks);
#pragma unroll
          for (int f = 0; f < FN; ++f)
#pragma unroll
            for (int g = 0; g < FM; ++g)
              acc[f][g] = mfma32<MODE>(wf[cb][f], af[cb][g], acc[f][g]);
        }
      }
    };

    // Stage kt % S holds K tile kt (the item's first S-1 tiles were issued before
    // it started, then the next item's row-index loads). Before reading a stage a
    // wavefront waits until at most the loads issued after that tile's are
    // outstanding. Loads complete in issue order among themselves, so this is exact
    // for the loads; stores in flight (the previous item's outputs) only hold the
    // count up, never let it pass early.
    for (int kt = 0; kt < cur.nk; ++kt) {
      const int ahead = min(S - 2, cur.nk - 1 - kt);  // tiles issued after kt
      if (ahead <= 0) wait_vmcnt<0>();
      else wait_vmcnt_upto<J * (S - 2) + JA>(J * ahead + (kt < S - 1 ? na : 0));
      stage_barrier();
      const int nt = kt + S - 1;  // K tile whose loads this step issues
      const int kvalid = cur.Kdim - kt * BK;
      if (kvalid < BK) {  // ragged last K tile: zero its chunks past k_dim (k_dim % 8 == 0)
        bf16_t* stg = smem + (kt % S) * STAGE;
        const int c0 = kvalid / 8, nc = CPR - c0;
        for (int i = tid; i < (BM + BN) * nc; i += 64 * NW)
          *reinterpret_cast<u32x4_t*>(&stg[lds_off<BK>(i / nc, c0 + i % nc)]) = u32x4_t{0, 0, 0, 0};
        stage_barrier();
      }
      if (!cur.wact) {
        issue(cur, nt, nt % S, -1);
        continue;
      }
      compute(std::true_type{}, kt % S, nt);
    }

    // Every wavefront is done with the stages: issue the next item's first tiles,
    // then store this item's outputs while those loads are in flight.
    const bool second = cur.second, wact = cur.wact;
    const int m0 = cur.m0, rows_valid = cur.rows_valid, col0 = cur.col0;
    stage_barrier();
    if (more) {
      setup(pre, cur);
      prologue(cur);
    }
    if (!wact) continue;
    const GemmProblem pr = second ? p1 : p0;
    const int Nout = pr.n_out;
    // epilogue: lane owns row l32 of each 32-row subtile, 4 consecutive columns per group
#pragma unroll
    for (int g = 0; g < FM; ++g) {
      const int rl = wm * TM + g * 32 + l32;
      if (rl >= rows_valid) continue;
      if (MODE == kSwiGLU) {
        bf16_t* crow = static_cast<bf16_t*>(pr.out) + (int64_t)(m0 + rl) * Nout;
#pragma unroll
        for (int f = 0; f < FN / 2; ++f)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int col = col0 + wn * (TN / 2) + f * 32 + 8 * q + 4 * half;
            if (col < Nout) {
              float h[4];
#pragma unroll
              for (int j = 0; j < 4; ++j)
                h[j] = silu(acc[f][g][4 * q + j]) * acc[f + FN / 2][g][4 * q + j];
              *reinterpret_cast<u32x2_t*>(crow + col) =
                  u32x2_t{pack_f16x2(h[0], h[1]), pack_f16x2(h[2], h[3])};
            }
          }
      } else {
        float* crow = static_cast<float*>(pr.out) + (int64_t)(m0 + rl) * Nout;
#pragma unroll
        for (int f = 0; f < FN; ++f)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int col = col0 + wn * TN + f * 32 + 8 * q + 4 * half;
            if (col < Nout) {
              const f32x16_t& v = acc[f][g];
              *reinterpret_cast<f32x4_t*>(crow + col) =
                  f32x4_t{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
            }
          }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Large tiles for MFMA-bound shapes: 256 activation rows x 256 weight rows x 32 K
// per tile, eight wavefronts in two groups of four that take turns ("ping-pong"):
// while one group's wavefronts run their MFMAs from registers, the other group's
// read their next fragments from LDS and issue global->LDS loads, and a workgroup
// barrier swaps the roles. With one wavefront of each group on every SIMD, the
// SIMD's matrix pipe always has a wavefront whose operands are in registers, and
// the LDS reads and the barrier waits of one group hide behind the other group's
// MFMAs instead of stalling all eight wavefronts at once.
//
// Per K tile a wavefront multiplies 128 activation rows by 64 weight rows (4 x 2
// blocks of v_mfma_f32_32x32x16, 16 MFMAs; 128 float32 accumulators): LDS reads of
// 0.75 KB per MFMA, and 64 KB of global->LDS loads feed 2^25 multiply-adds, 1.5x
// fewer bytes per FLOP than the 128 x 256 tile. Four LDS stages (128 KB) keep three
// K tiles in flight. Which wavefronts share a SIMD is read from the hardware (HW_ID)
// at kernel start; the group and the output block of each wavefront follow from it
// (if the placement is not two wavefronts per SIMD, wavefront w takes role w, which
// only costs speed).
//
// Phases, separated by barriers, for an item of nk K tiles (MEM(k): read tile k's
// fragments into registers; COMP(k): its 16 MFMAs):
//   group 0:        MEM(0) | COMP(0) | MEM(1) | COMP(1) | ... | COMP(nk-1) |
//   group 1:  ----- | MEM(0) | COMP(0) | MEM(1) | ...        | MEM(nk-1) | COMP(nk-1)
// Tile k's loads are issued in phase 2(k - 3) (group 0 in its MEM, group 1 before its
// MFMAs) into the stage tile k - 4 used, which every wavefront has read by then; each
// wavefront waits for its own loads of tile k before the barrier that opens phase 2k.
constexpr int kPpBM = 256, kPpBN = 256, kPpBK = 32, kPpS = 4, kPpNW = 8;

// K-major weight stages (kPlainKM): 1 KB piece i of a stage's weight region holds K rows
// 2i and 2i + 1 of the tile (BN weight rows of 2 bytes each); lanes 0-31 fill the first.
__device__ __forceinline__ int kmajor_krow(int i, int lane) { return 2 * i + (lane >> 5); }

// The four bf16 MFMA weight fragments of one K tile (two 16-wide K steps x two 32-row
// weight blocks) from a K-major weight stage [32 K rows][BN], by transposing LDS reads
// (ds_read_b64_tr_b16): within each 16-lane block the read gives lane i element i % 4
// of the 4-element pieces that lanes 4 j + i / 4 (j = 0..3) address, so lanes whose
// addresses walk K rows (lane / 4) and 4-column steps (lane % 4) each receive one
// column's four consecutive K values; two reads (K rows + 0..3, + 4..7) make a fragment.
// a0 / a1: the lane's LDS byte addresses (from the workgroup's LDS base) for weight
// blocks 0 / 1 at the tile's first K row; the K steps are 16 rows (16 BN 2 bytes) apart.
// Inline assembly because the compiler, which cannot tell these reads from the
// buffer->LDS loads still in flight, would otherwise wait for every outstanding load
// before them; the stage was waited for (and a barrier passed) before this call. All
// eight reads are issued before one wait for them inside the same statement, so no
// output register is seen before its read has landed.
typedef short s16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x8_t kmajor_pair(s16x4_t lo, s16x4_t hi) {
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}
// All twelve fragments of a K tile when both operands are K-major ([32 K rows][256],
// fragment layout [K step][two weight blocks, then four activation blocks]): addresses
// b0, b1 of the weight blocks and a0..a3 of the activation blocks, as kmajor_frags.
template <int BM>
__device__ __forceinline__ void kmajor_frags_all(uint32_t b0, uint32_t b1, uint32_t a0, uint32_t a1, uint32_t a2,
                                                 uint32_t a3, bf16x8_t (&fr)[2][6]) {
  static_assert(BM == 256, "offsets below: K step 16 rows (8192 bytes), half 4 rows (2048)");
  s16x4_t r[24];  // [K step][half][block]
  asm volatile(
      "ds_read_b64_tr_b16 %0, %24\n\t"
      "ds_read_b64_tr_b16 %1, %25\n\t"
      "ds_read_b64_tr_b16 %2, %26\n\t"
      "ds_read_b64_tr_b16 %3, %27\n\t"
      "ds_read_b64_tr_b16 %4, %28\n\t"
      "ds_read_b64_tr_b16 %5, %29\n\t"
      "ds_read_b64_tr_b16 %6, %24 offset:2048\n\t"
      "ds_read_b64_tr_b16 %7, %25 offset:2048\n\t"
      "ds_read_b64_tr_b16 %8, %26 offset:2048\n\t"
      "ds_read_b64_tr_b16 %9, %27 offset:2048\n\t"
      "ds_read_b64_tr_b16 %10, %28 offset:2048\n\t"
      "ds_read_b64_tr_b16 %11, %29 offset:2048\n\t"
      "ds_read_b64_tr_b16 %12, %24 offset:8192\n\t"
      "ds_read_b64_tr_b16 %13, %25 offset:8192\n\t"
      "ds_read_b64_tr_b16 %14, %26 offset:8192\n\t"
      "ds_read_b64_tr_b16 %15, %27 offset:8192\n\t"
      "ds_read_b64_tr_b16 %16, %28 offset:8192\n\t"
      "ds_read_b64_tr_b16 %17, %29 offset:8192\n\t"
      "ds_read_b64_tr_b16 %18, %24 offset:10240\n\t"
      "ds_read_b64_tr_b16 %19, %25 offset:10240\n\t"
      "ds_read_b64_tr_b16 %20, %26 offset:10240\n\t"
      "ds_read_b64_tr_b16 %21, %27 offset:10240\n\t"
      "ds_read_b64_tr_b16 %22, %28 offset:10240\n\t"
      "ds_read_b64_tr_b16 %23, %29 offset:10240\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7]),
        "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]), "=&v"(r[12]), "=&v"(r[13]), "=&v"(r[14]),
        "=&v"(r[15]), "=&v"(r[16]), "=&v"(r[17]), "=&v"(r[18]), "=&v"(r[19]), "=&v"(r[20]), "=&v"(r[21]),
        "=&v"(r[22]), "=&v"(r[23])
      : "v"(b0), "v"(b1), "v"(a0), "v"(a1), "v"(a2), "v"(a3));
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int blk = 0; blk < 6; ++blk) fr[ks][blk] = kmajor_pair(r[12 * ks + blk], r[12 * ks + 6 + blk]);
}
template <int BN>
__device__ __forceinline__ void kmajor_frags(uint32_t a0, uint32_t a1, bf16x8_t& f00, bf16x8_t& f01,
                                             bf16x8_t& f10, bf16x8_t& f11) {
  constexpr int kStep = 16 * BN * 2, kHalf = 4 * BN * 2;
  s16x4_t r[8];
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %8 offset:%10\n\t"
      "ds_read_b64_tr_b16 %2, %9\n\t"
      "ds_read_b64_tr_b16 %3, %9 offset:%10\n\t"
      "ds_read_b64_tr_b16 %4, %8 offset:%11\n\t"
      "ds_read_b64_tr_b16 %5, %8 offset:%12\n\t"
      "ds_read_b64_tr_b16 %6, %9 offset:%11\n\t"
      "ds_read_b64_tr_b16 %7, %9 offset:%12\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
      : "v"(a0), "v"(a1), "i"(kHalf), "i"(kStep), "i"(kStep + kHalf));
  f00 = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(r[0], r[1], 0, 1, 2, 3, 4, 5, 6, 7));
  f01 = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(r[2], r[3], 0, 1, 2, 3, 4, 5, 6, 7));
  f10 = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(r[4], r[5], 0, 1, 2, 3, 4, 5, 6, 7));
  f11 = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(r[6], r[7], 0, 1, 2, 3, 4, 5, 6, 7));
}

// The combine in the epilogue of the shared expert's down projection (kDownComb).
// The wavefront holds, in acc[f][g], rows rbase + 32 g + l32 (g < 4) of the tile and in
// each row the four-column groups c0 + 32 f + 8 q + 4 half (f < 2, q < 4) of the shared
// expert's float32 output. Token row t becomes bf16(acc_t + sum over k < n_t of
// w_tk z[t kr + k]), each term added with fmaf in slot order, as the standalone combine
// adds them. One row block at a time, slot after slot while any of its tokens has one
// left; a lane whose token has none left reads past the buffer's end (zero, no memory
// access) and keeps its sum. (Two blocks at a time, 16 loads in flight per lane, made
// the compiler spill.) The loop bound is uniform (a count of votes): a bound the
// compiler cannot see to be uniform made it spill the K loop's load offsets.
__device__ __forceinline__ void combine_epilogue(const GemmProblem& pr, int m0, int rows_valid, int rbase, int c0,
                                                 f32x16_t (&acc)[2][4]) {
  // (lane values derived here, behind opaque_v, so that nothing of this epilogue is
  // computed ahead of the K loop and held in registers through it)
  const int lane = opaque_v((int)threadIdx.x) & (kWave - 1), half = lane >> 5, l32 = lane & 31;
  const int Nout = pr.n_out, kk = pr.comb_k, kr = pr.comb_kr;
  const uint32_t z_end = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)pr.max_rows * kr * Nout * 4));
  const __amdgpu_buffer_rsrc_t rz = buffer_rsrc(uniform_ptr(pr.comb_z), z_end);
  int nk[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int rl = rbase + g * 32 + l32;
    nk[g] = rl < rows_valid ? min(max(pr.comb_n[m0 + rl], 0), kr) : 0;
  }
  const uint32_t cofs = (uint32_t)(c0 + 4 * half) * 4u;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int rl = rbase + g * 32 + l32, tok = m0 + rl;
    // (k < n_t <= min(K, N) <= K for every row that takes a term, so wrow[k] stays in
    // the row; rows past the tile's last read the tile's first)
    const float* wrow = pr.comb_w + (int64_t)(rl < rows_valid ? tok : m0) * kk;
    const uint32_t zrow = (uint32_t)tok * (uint32_t)kr * (uint32_t)Nout * 4u + cofs;
    // slots of the block: the most any of its tokens has (a count of wave-wide votes, so
    // the loop bound is uniform)
    int nmax = 0;
    for (int k = 0; k < kr; ++k) nmax += ballot(nk[g] > k) != 0;
    for (int k = 0; k < nmax; ++k) {
      const bool on = k < nk[g];
      const float w = wrow[k];
      const uint32_t rb = on ? zrow + (uint32_t)k * (uint32_t)Nout * 4u : z_end;
      f32x4_t z[2][4];
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          z[f][q] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rz, rb + (uint32_t)(f * 32 + 8 * q) * 4u, 0, 0));
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float a = acc[f][g][4 * q + j];
            acc[f][g][4 * q + j] = on ? fmaf(w, z[f][q][j], a) : a;
          }
    }
  }
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int rl = rbase + g * 32 + l32;
    if (rl >= rows_valid) continue;
    bf16_t* crow = static_cast<bf16_t*>(pr.out) + (int64_t)(m0 + rl) * Nout;
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = c0 + f * 32 + 8 * q + 4 * half;
        if (col < Nout) {
          const f32x16_t& v = acc[f][g];
          *reinterpret_cast<u32x2_t*>(crow + col) =
              u32x2_t{pack_bf16x2(v[4 * q], v[4 * q + 1]), pack_bf16x2(v[4 * q + 2], v[4 * q + 3])};
        }
      }
  }
}

constexpr size_t kPpLds = (size_t)kPpS * (kPpBM + kPpBN) * kPpBK * sizeof(bf16_t);  // 128 KB

// SIMD of the calling wavefront within its CU (HW_ID bits 5:4).
__device__ __forceinline__ int wave_simd() {
  return (int)__builtin_amdgcn_s_getreg(4 | (4 << 6) | ((2 - 1) << 11));
}

// Workgroup barrier that nothing is scheduled across (LDS reads retired first).
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  stage_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

template <int MODE, int ROLE>
__global__ void __launch_bounds__(64 * kPpNW) __attribute__((amdgpu_waves_per_eu(2, 2)))
grouped_gemm_pp_kernel(GemmProblem p0, GemmProblem p1) {
  constexpr int BM = kPpBM, BN = kPpBN, BK = kPpBK, S = kPpS, NW = kPpNW;
  constexpr bool SW = MODE == kSwiGLU || MODE == kSwiGLUKeep;  // gate and up weight halves
  constexpr int OC = SW ? BN / 2 : BN;  // output columns per tile
  constexpr int FM = 4, FN = 2;                      // 32-row blocks per wavefront: activations, weights
  constexpr bool KM = MODE == kPlainKM || MODE == kPlainKM2;  // K-major weights
  constexpr bool KMA = MODE == kPlainKM2;                      // and K-major activations
  constexpr bool ROWS = MODE == kDown16 && ROLE == 2; // output rows redirected (out_rows)
  constexpr int CPR = BK / 8, RPI = kWave / CPR;     // 16-byte chunks per row; rows per load instruction
  constexpr int J = (BM + BN) / (RPI * NW);          // load instructions per stage per wavefront (4)
  constexpr int JA = BM / (RPI * NW);                // of which fill activation rows (2)
  constexpr int STAGE = (BM + BN) * BK;
  static_assert(S == 4 && J == 4 && JA == 2, "the phase schedule below is written for this shape");
  __shared__ TileTable tt;
  __shared__ int simd_count[4];
  extern __shared__ __attribute__((aligned(16))) bf16_t smem[];  // [S][BM + BN][BK]
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  if (tid < 4) simd_count[tid] = 0;
  build_tile_table(tt, p0, p1, OC, BM);  // ends with a workgroup barrier
  const int simd = __builtin_amdgcn_readfirstlane(wave_simd()) & 3;
  int ord = 0;
  if (lane == 0) ord = atomicAdd(&simd_count[simd], 1);
  ord = __builtin_amdgcn_readfirstlane(__shfl(ord, 0, kWave));
  __syncthreads();
  // (read back through readfirstlane: the LDS values are the same in every lane, and the
  // compiler must know the role is wave-uniform or every branch on it becomes divergent)
  const int paired = __builtin_amdgcn_readfirstlane(
      simd_count[0] == 2 && simd_count[1] == 2 && simd_count[2] == 2 && simd_count[3] == 2);
  const int role = __builtin_amdgcn_readfirstlane(paired ? (ord & 1) * 4 + simd : wave);
  const int grp = role >> 2, wm = role & 1, wn = role >> 1;  // wn: weight quarter (group 0: 0, 1)
  const int G0 = p0.groups, G = p0.groups + p1.groups;
  const int total = tt.prefix[kMaxGroups];
  const int half = lane >> 5, l32 = lane & 31;
  // this lane's loads: row RPI (wave + NW j) + lrow of the stage, physical chunk lane % CPR,
  // logical chunk lc (the swizzle of lds_off<32>; each instruction's first row is a
  // multiple of 16)
  const int lrow = lane / CPR;
  const uint32_t lk = (uint32_t)(((lane % CPR) ^ ((lrow >> 2) & 3)) * 8);  // K column of the lane's chunk

  // XCD-contiguous tile ranges with the last round split by output columns, as in
  // the 128 x 256 kernel (here into halves or quarters of the four weight quarters).
  const int P = gridDim.x;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int Bx = P >> 3;
  const int T0 = tt.prefix[G0], T1 = total - T0;
  const int b0 = (int)((int64_t)xcd * T0 / 8), n0 = (int)((int64_t)(xcd + 1) * T0 / 8) - b0;
  const int b1 = T0 + (int)((int64_t)xcd * T1 / 8), n1 = T0 + (int)((int64_t)(xcd + 1) * T1 / 8) - b1;
  const int nx = n0 + n1;
  const int full = nx / Bx * Bx, rem = nx - full;
  const int split = rem == 0 ? 1 : (4 * rem <= Bx) ? 4 : (2 * rem <= Bx) ? 2 : 1;
  const int items = full + rem * split;

  // One work item, every field wave-uniform.
  struct Where {
    int second, ge, Kdim, kofs, nk, m0, rows_valid, col0, parts;
  };
  auto locate = [&](int it, Where& w) {
    int i = it, part = 0, parts = 1;
    if (it >= full) {
      i = full + (it - full) / split;
      part = (it - full) % split;
      parts = split;
    }
    const int L = i < n1 ? b1 + i : b0 + (i - n1);
    int lo = 0, hi = G;  // prefix[lo] <= L < prefix[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (tt.prefix[mid] <= L) lo = mid; else hi = mid;
    }
    const int e = __builtin_amdgcn_readfirstlane(lo);
    w.second = e >= G0;
    w.ge = w.second ? e - G0 : e;
    w.Kdim = __builtin_amdgcn_readfirstlane(tt.klen[e]);
    w.kofs = __builtin_amdgcn_readfirstlane(tt.kofs[e]);
    w.nk = (w.Kdim + BK - 1) / BK;
    const int local = L - __builtin_amdgcn_readfirstlane(tt.prefix[e]);
    int mtile, ntile;
    tile_of(w.second ? p1 : p0, local, __builtin_amdgcn_readfirstlane(tt.mt[e]),
            __builtin_amdgcn_readfirstlane(tt.nt[e]), mtile, ntile);
    w.m0 = __builtin_amdgcn_readfirstlane(tt.start[e] + mtile * BM);
    w.rows_valid = __builtin_amdgcn_readfirstlane(min(BM, tt.start[e] + tt.len[e] - w.m0));
    w.parts = parts;
    w.col0 = ntile * OC + part * (OC / parts);
  };
  // Row indices of this lane's activation loads for item w: gathered problems read
  // them from a_rows (global loads left in flight).
  auto fetch_rows = [&](const Where& w, int (&arow)[JA]) {
    const GemmProblem pr = w.second ? p1 : p0;
#pragma unroll
    for (int j = 0; j < JA; ++j) {
      const int r = RPI * (wave + NW * j) + lrow;
      arow[j] = w.m0 + (r < w.rows_valid ? r : 0);
    }
    if (pr.a_rows) {
#pragma unroll
      for (int j = 0; j < JA; ++j) arow[j] = pr.a_rows[arow[j]];
    }
  };
  // Operand resources and this lane's row offsets for item w. Rows past the segment
  // and weight rows outside the item's output columns point one row past their
  // resource's end: their loads read zero without touching memory.
  struct Tile {
    __amdgpu_buffer_rsrc_t ra, rb0, rb1;
    uint32_t a_end, b_end;
    uint32_t off[J];
    uint32_t b_row;  // K-major weights: bytes per K row
    int k_split;     // K-major weights: K rows read from rb0 (the rest from rb1)
    uint32_t a_row;  // K-major activations: bytes per K row
  };
  auto setup = [&](const Where& w, const int (&arow)[JA], Tile& t) {
    const GemmProblem pr = w.second ? p1 : p0;
    const int Nout = pr.n_out, ocp = OC / w.parts;
    const int64_t lda = pr.lda ? pr.lda : pr.k_dim, ldb = pr.ldb ? pr.ldb : pr.k_dim;
    const uint32_t a_rb = (uint32_t)lda * 2, b_rb = (uint32_t)ldb * 2;
    const int64_t wofs = pr.k_offsets ? (int64_t)w.kofs : (int64_t)w.ge * Nout * ldb;
    const int64_t abase = pr.a_rows ? 0 : w.m0 - (pr.rows_per_group ? (int64_t)w.ge * pr.rows_per_group : 0);
    if constexpr (KMA) {
      // rows [kofs, kofs + klen) of the [rows][lda] activation source are the item's K;
      // its output rows are the columns abase + ... (rows past klen read zero)
      t.a_row = __builtin_amdgcn_readfirstlane(a_rb);
      t.a_end = __builtin_amdgcn_readfirstlane((uint32_t)w.Kdim * a_rb);
      t.ra = buffer_rsrc(uniform_ptr(pr.a + (int64_t)w.kofs * lda), t.a_end);
    } else {
      t.a_end = __builtin_amdgcn_readfirstlane((uint32_t)((pr.a_rows ? pr.a_nrows : w.rows_valid) * a_rb));
      t.ra = buffer_rsrc(uniform_ptr(pr.a + abase * lda + w.kofs), t.a_end);
    }
    if constexpr (KM) {
      if (pr.k_offsets) {
        // weight-gradient form: rows [kofs, kofs + klen) of the one [rows][ldb] matrix b0
        // (rows past klen read zero; no second matrix)
        t.b_row = __builtin_amdgcn_readfirstlane(b_rb);
        t.k_split = 0x7fffffff;
        t.b_end = __builtin_amdgcn_readfirstlane((uint32_t)w.Kdim * b_rb);
        t.rb0 = buffer_rsrc(uniform_ptr(pr.b0 + (int64_t)w.kofs * ldb), t.b_end);
        t.rb1 = t.rb0;
      } else {
        // group ge's [k_split][Nout] matrix of b0 and [k_dim - k_split][Nout] matrix of b1;
        // one end (the larger matrix) serves both, every K row a lane reads being inside its own
        const int k0 = pr.k_split, k1 = pr.k_dim - pr.k_split;
        t.b_row = __builtin_amdgcn_readfirstlane((uint32_t)Nout * 2u);
        t.k_split = __builtin_amdgcn_readfirstlane(k0);
        t.b_end = __builtin_amdgcn_readfirstlane((uint32_t)max(k0, k1) * t.b_row);
        t.rb0 = buffer_rsrc(uniform_ptr(pr.b0 + (int64_t)w.ge * k0 * Nout), t.b_end);
        t.rb1 = buffer_rsrc(uniform_ptr(k1 > 0 ? pr.b1 + (int64_t)w.ge * k1 * Nout : pr.b0), t.b_end);
      }
    } else {
      t.b_end = __builtin_amdgcn_readfirstlane((uint32_t)Nout * b_rb);
      t.rb0 = buffer_rsrc(uniform_ptr(pr.b0 + wofs), t.b_end);
      t.rb1 = buffer_rsrc(uniform_ptr(SW ? pr.b1 + wofs : pr.b0 + wofs), t.b_end);
    }
#pragma unroll
    for (int j = 0; j < JA; ++j) {
      if constexpr (KMA) {
        // piece i of the activation region: K rows 2i, 2i + 1 of 256 output rows each,
        // swizzled as the weight region
        const int krow = kmajor_krow(wave + NW * j, lane);
        const int p16 = lane & 31;
        const int c = ((p16 & 3) | (((p16 >> 2) ^ (krow & 3)) << 2)) * 8;
        t.off[j] = c < w.rows_valid ? (uint32_t)krow * a_rb + (uint32_t)(abase + c) * 2u : t.a_end;
      } else {
        const int r = RPI * (wave + NW * j) + lrow;
        const int64_t row = pr.a_rows ? min<int64_t>(max<int64_t>(arow[j], 0), pr.a_nrows - 1) : r;
        t.off[j] = (r >= w.rows_valid ? t.a_end : (uint32_t)row * a_rb) + lk * 2;
      }
    }
#pragma unroll
    for (int j = JA; j < J; ++j) {
      if constexpr (KM) {
        // 1 KB piece i of the stage's weight region holds K rows 2i and 2i + 1 (512 bytes
        // each: 256 weight rows); the lane fills physical 16-byte chunk lane % 32 of its
        // row with the logical chunk the swizzle of the fragment reads places there (the
        // 64-byte column groups XOR-ed with k % 4)
        const int krow = kmajor_krow(wave + NW * (j - JA), lane);
        const int p16 = lane & 31;
        const int c = ((p16 & 3) | (((p16 >> 2) ^ (krow & 3)) << 2)) * 8;
        const int n = w.col0 + c;
        t.off[j] = c < ocp && n < Nout ? (uint32_t)krow * t.b_row + (uint32_t)n * 2u : t.b_end;
      } else {
        const int r = RPI * (wave + NW * j) + lrow - BM;
        const int c = SW ? r % OC : r;
        const int n = w.col0 + c;
        t.off[j] = (c < ocp && n < Nout ? (uint32_t)n * b_rb : t.b_end) + lk * 2;
      }
    }
  };
  // This wavefront's J loads of K tile kt into stage st. Chunks past the K range,
  // and every chunk of a tile past the item's last, read past their resource's end
  // (zero, no memory access), so no LDS fix-up is needed and every wavefront issues J
  // loads per tile slot, which keeps the wait counts constant. (A tile past the end
  // lands in a stage that nothing reads before this wavefront's own later loads
  // refill it.)
  auto issue = [&](const Tile& t, const Where& w, int kt, int st) {
    const uint32_t kb = (uint32_t)kt * (BK * 2);
    const bool in = kt < w.nk && (int)(kt * BK + lk) < w.Kdim;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      if (KMA && j < JA) {
        // K rows [kt BK, kt BK + BK) of the activation source (past klen: zero)
        buffer_load_lds16(t.ra, kt < w.nk ? t.off[j] + (uint32_t)(kt * BK) * t.a_row : t.a_end,
                          smem + st * STAGE + RPI * (wave + NW * j) * BK);
        continue;
      }
      if (KM && j >= JA) {
        // K rows [kt BK, kt BK + BK) of the weights: from rb0 below k_split, else rb1
        // (k_split and k_dim are multiples of BK, so a tile is whole and never straddles)
        const int kg = kt * BK;
        const bool second = kg >= t.k_split;
        const uint32_t kbw = (uint32_t)(second ? kg - t.k_split : kg) * t.b_row;
        buffer_load_lds16(second ? t.rb1 : t.rb0, kt < w.nk ? t.off[j] + kbw : t.b_end,
                          smem + st * STAGE + RPI * (wave + NW * j) * BK);
        continue;
      }
      const bool up = SW && j >= JA && RPI * (wave + NW * j) - BM >= OC;
      const uint32_t end = j < JA ? t.a_end : t.b_end;
      buffer_load_lds16(j < JA ? t.ra : up ? t.rb1 : t.rb0, in ? t.off[j] + kb : end,
                        smem + st * STAGE + RPI * (wave + NW * j) * BK);
    }
  };
  // Stages rotate across items: K tile kt of an item lives in stage (sb + kt) % S,
  // where sb advances by the item's tile count, so the next item's first tiles never
  // land in the stage of the current item's last tile, which group 1 still reads
  // after the last barrier.
  auto prologue = [&](const Tile& t, const Where& w, int sb) {
#pragma unroll
    for (int s = 0; s < S - 1; ++s) issue(t, w, s, (sb + s) & (S - 1));
  };

  // Fragment addresses: one per-lane byte offset per 16-wide K step for the first
  // activation block and the first weight block; the other blocks of the same K step
  // are whole 32-row strides further on (the swizzle term (row / 4) % 4 repeats every
  // 32 rows), so they fold into the LDS reads' immediate offsets.
  uint32_t a_lane[KMA ? 4 : 2], b_lane[2];
  if constexpr (KMA) {
    // K-major activation region [BK][BM]: a_lane[g] addresses the wavefront's 32-row
    // block g (rows wm BM / 2 + 32 g ...) as b_lane does the weight blocks below
    const int s16 = lane & 15;
    const int kl = 8 * (lane >> 5) + (s16 >> 2), nl = 16 * ((lane >> 4) & 1) + 4 * (s16 & 3);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int chunk = 4 * wm + g;
      a_lane[g] = (uint32_t)(kl * BM + ((chunk ^ (kl & 3)) * 32) + nl) * 2;
    }
  }
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    if constexpr (!KMA) a_lane[ks] = (uint32_t)lds_off<BK>(wm * (BM / 2) + l32, ks * 2 + half) * 2;
    if constexpr (KM) {
      // K-major weight region [BK][BN]: here b_lane[f] is the lane's transposing-read
      // address of weight block f (rows wn 64 + 32 f ...), K step and half folded into
      // immediates (their K offsets are multiples of 4, so the swizzle term k % 4 is the
      // lane's own). Lane l of each 16-lane block b addresses K row 8 (b / 2) + (l % 16) / 4
      // and weight rows 16 (b % 2) + 4 (l % 4) .. + 3 of the block; the read hands lane l
      // the four K values of weight row l % 32 (the MFMA's fragment layout).
      const int s16 = lane & 15;
      const int kl = 8 * (lane >> 5) + (s16 >> 2), nl = 16 * ((lane >> 4) & 1) + 4 * (s16 & 3);
      const int chunk = 2 * wn + ks;  // the wavefront's 32-row weight block ks
      b_lane[ks] = (uint32_t)(BM * BK + kl * BN + ((chunk ^ (kl & 3)) * 32) + nl) * 2;
    } else {
      b_lane[ks] = (uint32_t)(BM * BK + lds_off<BK>((SW ? wn * 32 : wn * 64) + l32, ks * 2 + half)) * 2;
    }
  }
  constexpr uint32_t kRow32 = 32 * BK * 2;                                   // bytes between 32-row blocks
  constexpr uint32_t kWStep = SW ? (BN / 2) * BK * 2 : kRow32;  // gate -> up, or block -> block
  typedef bf16x8_t Frags[2][FN + FM];  // per 16-wide K step: FN weight fragments, then FM activation ones
  auto read_frags = [&](int st, Frags& fr) {
    const char* base = reinterpret_cast<const char*>(smem) + st * (STAGE * 2);
    if constexpr (KMA) {
      // LDS byte address of the stage (the dynamic LDS follows the static tile table)
      const uint32_t sb = (uint32_t)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)base);
      kmajor_frags_all<BM>(sb + b_lane[0], sb + b_lane[1], sb + a_lane[0], sb + a_lane[1], sb + a_lane[2],
                           sb + a_lane[3], fr);
      return;
    } else if constexpr (KM) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int g = 0; g < FM; ++g)
          fr[ks][FN + g] = *reinterpret_cast<const bf16x8_t*>(base + a_lane[ks] + g * kRow32);
      // LDS byte address of the stage (the dynamic LDS follows the static tile table)
      const uint32_t sb = (uint32_t)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)base);
      kmajor_frags<BN>(sb + b_lane[0], sb + b_lane[1], fr[0][0], fr[0][1], fr[1][0], fr[1][1]);
      return;
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int f = 0; f < FN; ++f) fr[ks][f] = *reinterpret_cast<const bf16x8_t*>(base + b_lane[ks] + f * kWStep);
#pragma unroll
      for (int g = 0; g < FM; ++g)
        fr[ks][FN + g] = *reinterpret_cast<const bf16x8_t*>(base + a_lane[ks] + g * kRow32);
    }
    // half-precision down projections: the weight fragments are widened to half here,
    // in place, so the MFMA phase needs no registers for converted copies
    if constexpr (MODE == kDown16 || MODE == kDownComb) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int f = 0; f < FN; ++f) fr[ks][f] = __builtin_bit_cast(bf16x8_t, bf16x8_to_f16x8(fr[ks][f]));
    }
  };
  // One MFMA of a multiplied K tile; the half-precision modes' weight fragments arrive
  // already widened (read_frags).
  auto mfma_pp = [](bf16x8_t w, bf16x8_t a, f32x16_t c) {
    if constexpr (MODE == kDown16 || MODE == kDownComb)
      return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, w), __builtin_bit_cast(f16x8_t, a), c,
                                                    0, 0, 0);
    else
      return __builtin_amdgcn_mfma_f32_32x32x16_bf16(w, a, c, 0, 0, 0);
  };

  if (slot >= items) return;
  Where cur, nxt;
  Tile tl;
  int rows[JA];
  int sb = 0;
  locate(slot, cur);
  fetch_rows(cur, rows);
  setup(cur, rows, tl);
  prologue(tl, cur, sb);
  // The next item's row indices are loaded right behind the current item's first
  // tiles; the K loop's waits (at most 2J of this wavefront's loads outstanding)
  // cover them by the third tile, long before the next set-up reads them.
  const bool has_next0 = slot + Bx < items;
  if (has_next0) {
    locate(slot + Bx, nxt);
    fetch_rows(nxt, rows);
  }
  for (int it = slot; it < items; it += Bx) {
    const bool more = it + Bx < items;
    const int nk = cur.nk;
    const bool wact = __builtin_amdgcn_readfirstlane(wn < 4 / cur.parts && wm * (BM / 2) < cur.rows_valid);
    f32x16_t acc[FN][FM];
#pragma unroll
    for (int f = 0; f < FN; ++f)
#pragma unroll
      for (int g = 0; g < FM; ++g) acc[f][g] = f32x16_t{};
    // A computing wavefront runs at raised issue priority, so that on its SIMD the
    // other group's LDS reads and loads fill the gaps between its MFMAs rather than
    // delay them (measured +4% on a dense GEMM).
    auto compute = [&](const Frags& fr) {
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int f = 0; f < FN; ++f)
#pragma unroll
          for (int g = 0; g < FM; ++g) acc[f][g] = mfma_pp(fr[ks][f], fr[ks][FN + g], acc[f][g]);
      __builtin_amdgcn_s_setprio(0);
    };
    // Before the barrier that opens tile kt's first read: this wavefront's loads of
    // tile kt have landed. Loads complete in issue order, and at most the loads of
    // tiles kt + 1 and kt + 2 (and the next item's row indices, before tile 3's) were
    // issued after them: wait until at most 2J are outstanding (stores only hold the
    // count up).
    auto wait_tile = [&]() { wait_vmcnt<2 * J>(); };
    auto st_of = [&](int kt) { return (sb + kt) & (S - 1); };
    // MEM(k): issue tile k + 3's loads (into the stage of tile k - 1, which both groups
    // have read by then), then read all of tile k's fragments into registers; COMP(k):
    // tile k's 32 MFMAs from registers only. Loads are issued only in MEM phases, so the
    // computing group never waits on the address unit.
    Frags fr;
    if (nk == 0) {
      // an empty K range (a weight gradient's segment without rows): the outputs are
      // zero; the prologue's loads (zero-fills of this wavefront's own stage rows) land
      // before the next item's loads of the same rows are issued
      wait_vmcnt<0>();
    } else if (grp == 0) {
      wait_tile();
      phase_barrier();
      for (int kt = 0; kt < nk; ++kt) {
        issue(tl, cur, kt + S - 1, st_of(kt + S - 1));  // MEM(kt)
        if (wact) read_frags(st_of(kt), fr);
        phase_barrier();
        if (wact) compute(fr);                           // COMP(kt)
        wait_tile();                                     // tile kt + 1
        phase_barrier();
      }
    } else {
      wait_tile();
      phase_barrier();
      phase_barrier();                                   // phase 0
      for (int kt = 0; kt < nk; ++kt) {
        issue(tl, cur, kt + S - 1, st_of(kt + S - 1));  // MEM(kt)
        if (wact) read_frags(st_of(kt), fr);
        wait_tile();                                     // tile kt + 1
        phase_barrier();
        if (kt + 1 == nk) break;                         // COMP(nk-1) comes after the loop
        if (wact) compute(fr);                           // COMP(kt)
        phase_barrier();
      }
      if (wact) compute(fr);                             // COMP(nk-1)
    }
    // Start the next item's first K tiles, then store this item's outputs. Every LDS
    // read of this item is done (group 1's last step multiplies from registers) and
    // the next item's tiles go to other stages. Issued first, the loads' latency passes
    // while the stores drain (loads and stores complete in issue order, so the next
    // item's first wait still covers both).
    // (The set-up is computed again after the stores rather than kept: holding its
    // offsets across the epilogue makes the register allocator spill.)
    const int sb_next = (sb + nk) & (S - 1);
    if (more) {
      Tile t1;
      setup(nxt, rows, t1);
      prologue(t1, nxt, sb_next);
    }
    if constexpr (MODE == kDownComb) {
      if (wact) combine_epilogue(cur.second ? p1 : p0, cur.m0, cur.rows_valid, wm * (BM / 2), cur.col0 + wn * 64, acc);
    } else if (wact) {
      const GemmProblem pr = cur.second ? p1 : p0;
      const int Nout = pr.n_out, m0 = cur.m0, rows_valid = cur.rows_valid, col0 = cur.col0;
#pragma unroll
      for (int g = 0; g < FM; ++g) {
        const int rl = wm * (BM / 2) + g * 32 + l32;
        if (rl >= rows_valid) continue;
        if (MODE == kSwiGLU) {
          bf16_t* crow = static_cast<bf16_t*>(pr.out) + (int64_t)(m0 + rl) * Nout;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int col = col0 + wn * 32 + 8 * q + 4 * half;
            if (col < Nout) {
              float h[4];
#pragma unroll
              for (int j = 0; j < 4; ++j) h[j] = silu(acc[0][g][4 * q + j]) * acc[1][g][4 * q + j];
              *reinterpret_cast<u32x2_t*>(crow + col) = u32x2_t{pack_f16x2(h[0], h[1]), pack_f16x2(h[2], h[3])};
            }
          }
        } else if (MODE == kSwiGLUKeep) {
          const int64_t ro = (int64_t)(m0 + rl) * Nout;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int col = col0 + wn * 32 + 8 * q + 4 * half;
            if (col < Nout) {
              const f32x4_t gv{acc[0][g][4 * q], acc[0][g][4 * q + 1], acc[0][g][4 * q + 2], acc[0][g][4 * q + 3]};
              const f32x4_t uv{acc[1][g][4 * q], acc[1][g][4 * q + 1], acc[1][g][4 * q + 2], acc[1][g][4 * q + 3]};
              *reinterpret_cast<u32x2_t*>(static_cast<bf16_t*>(pr.keep_g) + ro + col) =
                  u32x2_t{pack_f16x2(gv[0], gv[1]), pack_f16x2(gv[2], gv[3])};
              *reinterpret_cast<u32x2_t*>(static_cast<bf16_t*>(pr.keep_u) + ro + col) =
                  u32x2_t{pack_f16x2(uv[0], uv[1]), pack_f16x2(uv[2], uv[3])};
              float h[4];
#pragma unroll
              for (int j = 0; j < 4; ++j) h[j] = silu(gv[j]) * uv[j];
              *reinterpret_cast<u32x2_t*>(static_cast<bf16_t*>(pr.out) + ro + col) =
                  u32x2_t{pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3])};
              if (pr.keep_h16)
                *reinterpret_cast<u32x2_t*>(static_cast<bf16_t*>(pr.keep_h16) + ro + col) =
                    u32x2_t{pack_f16x2(h[0], h[1]), pack_f16x2(h[2], h[3])};
            }
          }
        } else {
          // routed rows of the layer go to their token-major slot rows (out_rows; compiled
          // only into the layer's down projection launch, since the load's wait would
          // also wait for the next item's first tiles, issued just before)
          const int64_t orow = ROWS && pr.out_rows ? (int64_t)pr.out_rows[m0 + rl] : (int64_t)(m0 + rl);
          float* crow = static_cast<float*>(pr.out) + orow * Nout;
#pragma unroll
          for (int f = 0; f < FN; ++f)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int col = col0 + wn * 64 + f * 32 + 8 * q + 4 * half;
              if (col < Nout) {
                const f32x16_t& v = acc[f][g];
                *reinterpret_cast<f32x4_t*>(crow + col) = f32x4_t{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
              }
            }
        }
      }
    }
    sb = sb_next;
    if (more) {
      cur = nxt;
#pragma unroll
      for (int j = 0; j < JA; ++j) rows[j] = opaque_v(rows[j]);
      setup(cur, rows, tl);
      if (it + 2 * Bx < items) {
        locate(it + 2 * Bx, nxt);
        fetch_rows(nxt, rows);
      }
    }
  }
}

// Few rows per group (decode-size token counts): the tiled kernel's work items are
// then a handful of weight panels, each a chain of latency-bound K steps. Here a
// work item is one group's 16 weight rows (16 gate + 16 up rows for SwiGLU) x up to
// 16 activation rows, the four wavefronts of a workgroup split K, every load goes
// straight to registers (all of a batch in flight at once) and feeds
// v_mfma_f32_16x16x32_bf16, and the four partial sums are added in LDS in wavefront
// order. Lane layout of that MFMA: lane l holds A[l % 16][8 (l / 16) + e] and
// B[8 (l / 16) + e][l % 16]; result register i is row 4 (l / 16) + i, column l % 16.
// A is the activation rows (m) and B the weight rows (n), transposed: B[k][j] =
// W[n0 + j][k]. Items are (group, 16-column block, 16-row block); a group with more
// than 16 rows takes several row blocks.
constexpr int kSkinnyRows = 16;
constexpr int kSkinnyBatch = 8;  // 32-wide K chunks loaded per batch

template <int MODE, int ROLE>
__global__ void __launch_bounds__(256)
skinny_gemm_kernel(GemmProblem p0, GemmProblem p1) {
  constexpr int NB = MODE == kSwiGLU ? 2 : 1;  // weight matrices per item
  __shared__ TileTable tt;
  __shared__ f32x4_t red[3][NB][kWave];
  build_tile_table(tt, p0, p1, kSkinnyRows, kSkinnyRows);
  const int G0 = p0.groups, G = p0.groups + p1.groups;
  const int total = tt.prefix[kMaxGroups];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int r16 = lane & 15, kq = lane >> 4;
  for (int L = blockIdx.x; L < total; L += gridDim.x) {
    int lo = 0, hi = G;  // prefix[lo] <= L < prefix[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (tt.prefix[mid] <= L) lo = mid; else hi = mid;
    }
    const int e = lo;
    const GemmProblem pr = e >= G0 ? p1 : p0;
    const int ge = e >= G0 ? e - G0 : e;
    const int Nout = pr.n_out, Kdim = pr.k_dim;
    const int local = L - tt.prefix[e];
    int mtile, ntile;
    tile_of(pr, local, tt.mt[e], tt.nt[e], mtile, ntile);
    const int m0 = tt.start[e] + mtile * kSkinnyRows;
    const int rows_valid = min(kSkinnyRows, tt.start[e] + tt.len[e] - m0);
    const int n0 = ntile * kSkinnyRows;
    // this lane's activation row and weight row (always valid rows; the extra rows
    // and columns only feed outputs that are never stored)
    int64_t arow = m0 + (r16 < rows_valid ? r16 : 0);
    if (pr.a_rows) arow = min<int64_t>(max<int64_t>(pr.a_rows[arow], 0), pr.a_nrows - 1);
    const bf16_t* ap = pr.a + arow * Kdim + 8 * kq;
    const int n = n0 + r16;
    const int64_t wrow = (int64_t)ge * Nout + (n < Nout ? n : 0);
    const bf16_t* bp[NB];
    bp[0] = pr.b0 + wrow * Kdim + 8 * kq;
    if constexpr (NB == 2) bp[1] = pr.b1 + wrow * Kdim + 8 * kq;
    // this wavefront's 32-wide K chunks
    const int nc = (Kdim + 31) / 32, per = (nc + 3) / 4;
    const int c0 = wave * per, c1 = min(nc, c0 + per);
    f32x4_t acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[b] = f32x4_t{};
    for (int c = c0; c < c1; c += kSkinnyBatch) {
      bf16x8_t av[kSkinnyBatch], bv[NB][kSkinnyBatch];  // kDown16: av holds half bits
#pragma unroll
      for (int j = 0; j < kSkinnyBatch; ++j) {
        const int k = (c + j) * 32 + 8 * kq;  // chunks of 8 are wholly inside or outside k_dim
        const bool in = c + j < c1 && k < Kdim;
        av[j] = in ? *reinterpret_cast<const bf16x8_t*>(ap + (c + j) * 32) : bf16x8_t{};
#pragma unroll
        for (int b = 0; b < NB; ++b)
          bv[b][j] = in ? *reinterpret_cast<const bf16x8_t*>(bp[b] + (c + j) * 32) : bf16x8_t{};
      }
#pragma unroll
      for (int j = 0; j < kSkinnyBatch; ++j)
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          if constexpr (MODE == kDown16)
            acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, av[j]),
                                                           bf16x8_to_f16x8(bv[b][j]), acc[b], 0, 0, 0);
          else
            acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[j], bv[b][j], acc[b], 0, 0, 0);
        }
    }
    if (wave > 0)
#pragma unroll
      for (int b = 0; b < NB; ++b) red[wave - 1][b][lane] = acc[b];
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int w = 0; w < 3; ++w) acc[b] += red[w][b][lane];
      const int col = n0 + r16;
      if (col < Nout) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = 4 * kq + i;
          if (m >= rows_valid) continue;
          const int64_t o = (int64_t)(m0 + m) * Nout + col;
          if constexpr (MODE == kSwiGLU) {
            static_cast<_Float16*>(pr.out)[o] = (_Float16)(silu(acc[0][i]) * acc[NB - 1][i]);
          } else {
            static_cast<float*>(pr.out)[o] = acc[0][i];
          }
        }
      }
    }
    __syncthreads();  // red is reused by the next item
  }
}

// float32 path: one thread per output element, plain FMA loops (small workloads).
template <int MODE>
__global__ void __launch_bounds__(256)
grouped_gemm_f32_kernel(const float* __restrict__ A, const int32_t* __restrict__ a_rows,
                        int64_t a_nrows, const int32_t* __restrict__ offsets, int groups,
                        int64_t max_rows, const float* __restrict__ B0,
                        const float* __restrict__ B1, int Nout, int Kdim, float* __restrict__ C) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= max_rows * Nout) return;
  const int64_t p = i / Nout;
  const int n = (int)(i - p * Nout);
  int e = -1;
  if (!offsets) {
    e = 0;
  } else {
    for (int g = 0; g < groups && e < 0; ++g) {
      const int64_t a = min<int64_t>(max<int64_t>((int64_t)offsets[g], 0), max_rows);
      const int64_t b = min<int64_t>(max<int64_t>((int64_t)offsets[g + 1], a), max_rows);
      if (p >= a && p < b) e = g;
    }
  }
  if (e < 0) return;
  const int64_t src = a_rows ? min<int64_t>(max<int64_t>(a_rows[p], 0), a_nrows - 1) : p;
  const float* arow = A + src * Kdim;
  const float* b0 = B0 + ((int64_t)e * Nout + n) * Kdim;
  float s0 = 0.0f;
  if (MODE == kSwiGLU) {
    const float* b1 = B1 + ((int64_t)e * Nout + n) * Kdim;
    float s1 = 0.0f;
    for (int k = 0; k < Kdim; ++k) {
      s0 = fmaf(arow[k], b0[k], s0);
      s1 = fmaf(arow[k], b1[k], s1);
    }
    C[p * Nout + n] = (s0 / (1.0f + expf(-s0))) * s1;
  } else {
    for (int k = 0; k < Kdim; ++k) s0 = fmaf(arow[k], b0[k], s0);
    C[p * Nout + n] = s0;
  }
}

// Tile shape: 128 rows x 256 weight rows on eight wavefronts (2 x 4, 64 x 64 each),
// three stages of 64-wide K tiles.
struct GemmShape {
  int bm, bn, threads;
  size_t lds;
};
template <int BM, int BN, int WM, int WN, int S, int BK>
constexpr GemmShape shape_of() {
  return GemmShape{BM, BN, 64 * WM * WN, (size_t)S * (BM + BN) * BK * sizeof(bf16_t)};
}

static unsigned gemm_grid(const GemmProblem& p0, const GemmProblem& p1, int bm, int oc,
                          int num_cus, int per_cu) {
  auto upper = [&](const GemmProblem& p) -> int64_t {
    if (p.groups == 0 || p.max_rows <= 0) return 0;
    return (p.max_rows / bm + p.groups) * ((p.n_out + oc - 1) / oc);
  };
  const int64_t tiles = upper(p0) + upper(p1);
  // persistent grid, a multiple of 8 (one contiguous tile range per XCD)
  const int cap = std::max(8, num_cus * per_cu / 8 * 8);
  return (unsigned)std::max<int64_t>(8, std::min<int64_t>(cap, (tiles + 7) / 8 * 8));
}

template <int MODE, int ROLE, int BM, int BN, int WM, int WN, int S, int BK>
static void launch_variant(const GemmProblem& q0, const GemmProblem& q1, int num_cus,
                           hipStream_t stream) {
  constexpr GemmShape sh = shape_of<BM, BN, WM, WN, S, BK>();
  static_assert(sh.lds + sizeof(TileTable) <= 160 * 1024, "LDS budget of one CU");
  constexpr int OC = MODE == kSwiGLU ? BN / 2 : BN;
  auto kern = grouped_gemm_bf16_kernel<MODE, ROLE, BM, BN, WM, WN, S, BK>;
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)sh.lds);
  // resident workgroups per CU (registers and LDS), queried once per instantiation
  static const int per_cu = [&] {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, sh.threads, sh.lds) != hipSuccess)
      n = 1;
    return std::max(1, std::min(n, 2));
  }();
  const unsigned grid = gemm_grid(q0, q1, BM, OC, num_cus, per_cu);
  kern<<<grid, sh.threads, sh.lds, stream>>>(q0, q1);
}

template <int MODE, int ROLE>
static void launch_pp(const GemmProblem& q0, const GemmProblem& q1, int num_cus, hipStream_t stream) {
  constexpr int OC = MODE == kSwiGLU ? kPpBN / 2 : kPpBN;
  auto kern = grouped_gemm_pp_kernel<MODE, ROLE>;
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)kPpLds);
  const unsigned grid = gemm_grid(q0, q1, kPpBM, OC, num_cus, 1);
  kern<<<grid, 64 * kPpNW, kPpLds, stream>>>(q0, q1);
}

// The 256 x 256 ping-pong tiles pay off when every problem of the launch has many
// rows per group (up to a quarter of a 256-row tile is lost per segment end): at
// least 512 rows per group if every slot were real (a routed problem's worst case,
// T min(K, N) rows over N experts; a dense problem's T). Plain forms only.
static bool use_pp(const GemmProblem& q0, const GemmProblem& q1) {
  auto ok = [](const GemmProblem& p) {
    if (p.groups == 0 || p.max_rows <= 0) return true;
    return (p.rows_per_group > 0 ? (int64_t)p.rows_per_group : p.max_rows / p.groups) >= 512;
  };
  return ok(q0) && ok(q1);
}

template <int MODE, int ROLE>
static void launch_shape(const GemmProblem& q0, const GemmProblem& q1, int num_cus, hipStream_t stream) {
  if (use_pp(q0, q1)) launch_pp<MODE, ROLE>(q0, q1, num_cus, stream);
  else launch_variant<MODE, ROLE, 128, 256, 2, 4, 3, 64>(q0, q1, num_cus, stream);
}

// Groups of at most this many rows take the skinny kernel (measured at the
// Qwen3-0.6B shape: T = 1 layer 53 -> 36 us; at 64 rows per group the tiled kernel
// is as fast, at 256 faster).
constexpr int64_t kSkinnyMaxRows = 32;
// Most rows any group of p can hold: a routed problem read through a_rows has at
// most one row per token and group.
static int64_t rows_per_group_bound(const GemmProblem& p) {
  if (p.groups == 0 || p.max_rows <= 0) return 0;
  return p.a_rows ? std::min(p.a_nrows, p.max_rows) : p.max_rows;
}

template <int MODE, int ROLE>
static void launch_skinny(const GemmProblem& q0, const GemmProblem& q1, int num_cus,
                          hipStream_t stream) {
  auto upper = [](const GemmProblem& p) -> int64_t {
    if (p.groups == 0 || p.max_rows <= 0) return 0;
    return (p.max_rows / kSkinnyRows + p.groups) * ((p.n_out + kSkinnyRows - 1) / kSkinnyRows);
  };
  const int64_t items = upper(q0) + upper(q1);
  const unsigned grid = (unsigned)std::max<int64_t>(1, std::min<int64_t>(items, 4 * (int64_t)num_cus));
  skinny_gemm_kernel<MODE, ROLE><<<grid, 256, 0, stream>>>(q0, q1);
}

bool gemm_operands_fit(const GemmProblem& p) {
  if (p.groups == 0 || p.max_rows <= 0) return true;
  const int64_t a_rb = (p.lda ? p.lda : p.k_dim) * 2, b_rb = (p.ldb ? p.ldb : p.k_dim) * 2;
  if (p.a_kmajor) return true;  // the K-major weight-gradient form checks its own offsets
  const int64_t b_bytes = p.b_kmajor ? (int64_t)(std::max(p.k_split, p.k_dim - p.k_split) + 1) * p.n_out * 2
                                     : (int64_t)(p.n_out + 1) * b_rb;
  return b_bytes <= 0xFFFFFFFFll &&
         (!p.a_rows || (p.a_nrows + 1) * a_rb <= 0xFFFFFFFFll) &&
         (!p.rows_per_group || (int64_t)(p.rows_per_group + 1) * a_rb <= 0xFFFFFFFFll);
}

static bool plain_form(const GemmProblem& p) { return !p.k_offsets && !p.lda && !p.ldb && !p.rows_per_group; }

// A K-major problem (op 1) the 256 x 256 kernel takes. Weights only: plain form
// otherwise, whole 8-column chunks per row, whole K tiles, the b0 / b1 boundary on a K
// tile boundary. Both operands (the weight-gradient form): per-group K ranges
// (k_offsets) of two row-major sources with 16-byte rows and 8-column chunks, their
// byte offsets (up to twice the K extent, the past-the-end reads included) within 4 GB.
static bool kmajor_ok(const GemmProblem& p) {
  if (p.groups == 0 || p.max_rows <= 0) return true;
  if (!p.b_kmajor || p.out_rows || p.n_out % 8 != 0) return false;
  if (p.a_kmajor) {
    const int64_t reach = 2 * (int64_t)p.k_dim + kPpBK;
    return p.k_offsets && !p.a_rows && !p.offsets && !p.b1 && p.rows_per_group > 0 && p.rows_per_group % 8 == 0 &&
           p.lda >= p.rows_per_group && p.lda % 8 == 0 && p.ldb >= p.n_out && p.ldb % 8 == 0 &&
           reach * p.lda * 2 <= 0xFFFFFFFFll && reach * p.ldb * 2 <= 0xFFFFFFFFll;
  }
  return plain_form(p) && p.k_split > 0 && p.k_split % kPpBK == 0 && p.k_dim % kPpBK == 0 &&
         p.k_split <= p.k_dim && (p.k_split < p.k_dim) == (p.b1 != nullptr);
}

static bool skinny_launch(const GemmProblem& q0, const GemmProblem& q1) {
  return plain_form(q0) && plain_form(q1) &&
         std::max(rows_per_group_bound(q0), rows_per_group_bound(q1)) <= kSkinnyMaxRows;
}

bool gemm_kmajor_ok(const GemmProblem& p0, const GemmProblem& p1) {
  const bool any0 = p0.groups > 0 && p0.max_rows > 0, any1 = p1.groups > 0 && p1.max_rows > 0;
  if (any0 && any1 && p0.a_kmajor != p1.a_kmajor) return false;
  return (!any0 || kmajor_ok(p0)) && (!any1 || kmajor_ok(p1)) && gemm_pair_uses_pp(p0, p1);
}

bool gemm_pair_uses_pp(const GemmProblem& p0, const GemmProblem& p1) {
  const bool any0 = p0.groups > 0 && p0.max_rows > 0, any1 = p1.groups > 0 && p1.max_rows > 0;
  const GemmProblem q0 = any0 ? p0 : GemmProblem{}, q1 = any1 ? p1 : GemmProblem{};
  return (any0 || any1) && !skinny_launch(q0, q1) && use_pp(q0, q1);
}

hipError_t launch_gemm_pair(bool bf16, int op, const GemmProblem& p0, const GemmProblem& p1,
                            int num_cus, hipStream_t stream, int role) {
  const bool any0 = p0.groups > 0 && p0.max_rows > 0, any1 = p1.groups > 0 && p1.max_rows > 0;
  if (!any0 && !any1) return hipSuccess;
  if (bf16 && (!gemm_operands_fit(p0) || !gemm_operands_fit(p1))) return hipErrorInvalidValue;
  if ((any0 ? p0.groups : 0) + (any1 ? p1.groups : 0) > kMaxGroups) return hipErrorInvalidValue;
  // the output-row redirect (the layer's down projection launch) and the combine
  // epilogue exist on the 256 x 256 tiles only
  const bool redirect = (any0 && p0.out_rows) || (any1 && p1.out_rows);
  if ((op == 3 || op == 4 || redirect) && (!bf16 || !gemm_pair_uses_pp(p0, p1))) return hipErrorInvalidValue;
  if (op == 4 && ((any0 && (!p0.keep_g || !p0.keep_u || p0.n_out % 4)) || (any1 && (!p1.keep_g || !p1.keep_u ||
                                                                                   p1.n_out % 4))))
    return hipErrorInvalidValue;
  if (redirect && (op != 2 || role != 2)) return hipErrorInvalidValue;
  const bool km = (any0 && p0.b_kmajor) || (any1 && p1.b_kmajor);
  if (km && (!bf16 || op != 1 || !gemm_kmajor_ok(p0, p1))) return hipErrorInvalidValue;
  if (bf16) {
    GemmProblem q0 = any0 ? p0 : GemmProblem{}, q1 = any1 ? p1 : GemmProblem{};
    if (km) {
      if ((any0 && p0.a_kmajor) || (any1 && p1.a_kmajor)) {
        if (role == 3) launch_pp<kPlainKM2, 3>(q0, q1, num_cus, stream);
        else launch_pp<kPlainKM2, 0>(q0, q1, num_cus, stream);
      } else {
        if (role == 3) launch_pp<kPlainKM, 3>(q0, q1, num_cus, stream);
        else launch_pp<kPlainKM, 0>(q0, q1, num_cus, stream);
      }
      return hipGetLastError();
    }
    if (op == 3) {
      if (role == 2) launch_pp<kDownComb, 2>(q0, q1, num_cus, stream);
      else return hipErrorInvalidValue;
      return hipGetLastError();
    }
    if (op == 4) {
      if (role == 3) launch_pp<kSwiGLUKeep, 3>(q0, q1, num_cus, stream);
      else if (role == 2) launch_pp<kSwiGLUKeep, 2>(q0, q1, num_cus, stream);
      else return hipErrorInvalidValue;
      return hipGetLastError();
    }
    if (skinny_launch(q0, q1)) {
#define MOE_SKINNY_DISPATCH(M_)                                            \
  do {                                                                     \
    if (role == 3) launch_skinny<M_, 3>(q0, q1, num_cus, stream);          \
    else if (role == 2) launch_skinny<M_, 2>(q0, q1, num_cus, stream);     \
    else if (role == 1) launch_skinny<M_, 1>(q0, q1, num_cus, stream);     \
    else launch_skinny<M_, 0>(q0, q1, num_cus, stream);                    \
  } while (0)
      if (op == 0) MOE_SKINNY_DISPATCH(kSwiGLU);
      else if (op == 2) MOE_SKINNY_DISPATCH(kDown16);
      else MOE_SKINNY_DISPATCH(kPlain);
#undef MOE_SKINNY_DISPATCH
      return hipGetLastError();
    }
#define MOE_GEMM_DISPATCH(M_)                                         \
  do {                                                                \
    if (role == 3) launch_shape<M_, 3>(q0, q1, num_cus, stream);      \
    else if (role == 2) launch_shape<M_, 2>(q0, q1, num_cus, stream); \
    else if (role == 1) launch_shape<M_, 1>(q0, q1, num_cus, stream); \
    else launch_shape<M_, 0>(q0, q1, num_cus, stream);                \
  } while (0)
    if (op == 0) MOE_GEMM_DISPATCH(kSwiGLU);
    else if (op == 2) MOE_GEMM_DISPATCH(kDown16);
    else MOE_GEMM_DISPATCH(kPlain);
#undef MOE_GEMM_DISPATCH
  } else {
    for (const GemmProblem* p : {&p0, &p1}) {
      if (p->groups == 0 || p->max_rows <= 0) continue;
      const int64_t n = p->max_rows * p->n_out;
      const unsigned grid = (unsigned)((n + 255) / 256);
      const float* A = reinterpret_cast<const float*>(p->a);
      if (op == 0)  // (op 2, the half-precision down projection, is op 1 for float32)
        grouped_gemm_f32_kernel<kSwiGLU><<<grid, 256, 0, stream>>>(
            A, p->a_rows, p->a_nrows, p->offsets, p->groups, p->max_rows,
            reinterpret_cast<const float*>(p->b0), reinterpret_cast<const float*>(p->b1), p->n_out,
            p->k_dim, static_cast<float*>(p->out));
      else
        grouped_gemm_f32_kernel<kPlain><<<grid, 256, 0, stream>>>(
            A, p->a_rows, p->a_nrows, p->offsets, p->groups, p->max_rows,
            reinterpret_cast<const float*>(p->b0), nullptr, p->n_out, p->k_dim,
            static_cast<float*>(p->out));
    }
  }
  return hipGetLastError();
}

hipError_t launch_expert_ffn(const FfnArgs& a, hipStream_t stream) {
  if (a.max_rows <= 0) return hipSuccess;
  GemmProblem none{};
  GemmProblem g1{static_cast<const bf16_t*>(a.a), nullptr, a.max_rows, a.offsets, a.groups,
                 a.max_rows, static_cast<const bf16_t*>(a.w_gate),
                 static_cast<const bf16_t*>(a.w_up), a.d_ff, a.d_model, a.h};
  const int role = a.offsets ? 0 : 1;
  hipError_t e = launch_gemm_pair(a.bf16, 0, g1, none, a.num_cus, stream, role);
  if (e != hipSuccess) return e;
  GemmProblem g2{static_cast<const bf16_t*>(a.h), nullptr, a.max_rows, a.offsets, a.groups,
                 a.max_rows, static_cast<const bf16_t*>(a.w_down), nullptr, a.d_model, a.d_ff,
                 a.out};
  return launch_gemm_pair(a.bf16, 2, g2, none, a.num_cus, stream, role);
}

}  // namespace moe
