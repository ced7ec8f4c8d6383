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
//    (expert, column tile, row tile); each problem's list is cut into 8 contiguous
//    ranges, one per XCD (workgroups are dispatched round-robin over the 8 XCDs),
//    so the row tiles that share one expert's weight panel run on the same L2 and
//    the shared expert's tiles are spread over all XCDs.
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

enum { kSwiGLU = 0, kPlain = 1 };

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

// Table of (group, column tile, row tile) over problem 0's groups followed by
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
        const GemmProblem& pr = e < G0 ? p0 : p1;
        const int ge = e < G0 ? e : e - G0;
        kl = pr.k_dim;
        if (pr.k_offsets) {
          ko = pr.k_offsets[ge];
          kl = max(0, pr.k_offsets[ge + 1] - ko);
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
  // Locates work item it (group, column tile, row tile, sub-tile columns), decides
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
    const int mt = tt.mt[e];
    const int ntile = local / mt, mtile = local - ntile * mt;
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
              acc[f][g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa[ks][f], aa[ks][g], acc[f][g], 0, 0, 0);
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
              acc[f][g] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[cb][f], af[cb][g], acc[f][g], 0, 0, 0);
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
                  u32x2_t{pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3])};
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
    const int mt = tt.mt[e];
    const int ntile = local / mt, mtile = local - ntile * mt;
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
      bf16x8_t av[kSkinnyBatch], bv[NB][kSkinnyBatch];
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
        for (int b = 0; b < NB; ++b)
          acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[j], bv[b][j], acc[b], 0, 0, 0);
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
            static_cast<bf16_t*>(pr.out)[o] = f32_to_bf16(silu(acc[0][i]) * acc[NB - 1][i]);
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

// Tile shape (BM x BN, wavefronts, stages, K tile): 128 x 256 on eight wavefronts,
// three stages of 64-wide K tiles. It measured fastest at both ends of the
// rows-per-expert range (64 and 512) among 128 x 128, 64 x 256, 128 x 384 (two
// stages, or four of 32-wide K tiles) and 128 x 256 with five 32-wide stages;
// those are compiled only for tuning builds (-DMOE_GEMM_VARIANT=k).
struct GemmShape {
  int bm, bn, threads;
  size_t lds;
};
template <int BM, int BN, int WM, int WN, int S, int BK>
constexpr GemmShape shape_of() {
  return GemmShape{BM, BN, 64 * WM * WN, (size_t)S * (BM + BN) * BK * sizeof(bf16_t)};
}

#ifndef MOE_GEMM_VARIANT
#define MOE_GEMM_VARIANT 0
#endif

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
static void launch_shape(int variant, const GemmProblem& q0, const GemmProblem& q1, int num_cus,
                         hipStream_t stream) {
  switch (variant) {
#if MOE_GEMM_VARIANT
    case 1: launch_variant<MODE, ROLE, 128, 128, 2, 2, 4, 64>(q0, q1, num_cus, stream); break;
    case 2: launch_variant<MODE, ROLE, 128, 256, 2, 2, 3, 64>(q0, q1, num_cus, stream); break;
    case 3: launch_variant<MODE, ROLE, 64, 256, 1, 4, 3, 64>(q0, q1, num_cus, stream); break;
    case 5: launch_variant<MODE, ROLE, 128, 384, 2, 2, 2, 64>(q0, q1, num_cus, stream); break;
    case 6: launch_variant<MODE, ROLE, 128, 384, 2, 2, 4, 32>(q0, q1, num_cus, stream); break;
    case 7: launch_variant<MODE, ROLE, 128, 256, 2, 4, 5, 32>(q0, q1, num_cus, stream); break;
    case 8: launch_variant<MODE, ROLE, 256, 256, 2, 2, 4, 32>(q0, q1, num_cus, stream); break;
    case 9: launch_variant<MODE, ROLE, 256, 256, 2, 2, 2, 64>(q0, q1, num_cus, stream); break;
    case 10: launch_variant<MODE, ROLE, 128, 256, 2, 4, 6, 32>(q0, q1, num_cus, stream); break;
    case 11: launch_variant<MODE, ROLE, 128, 256, 2, 4, 4, 32>(q0, q1, num_cus, stream); break;
    case 12: launch_variant<MODE, ROLE, 256, 256, 2, 4, 2, 64>(q0, q1, num_cus, stream); break;
    case 13: launch_variant<MODE, ROLE, 256, 256, 4, 2, 2, 64>(q0, q1, num_cus, stream); break;
    case 14: launch_variant<MODE, ROLE, 128, 128, 2, 2, 2, 64>(q0, q1, num_cus, stream); break;
    case 15: launch_variant<MODE, ROLE, 128, 128, 2, 2, 3, 32>(q0, q1, num_cus, stream); break;
    case 16: launch_variant<MODE, ROLE, 256, 256, 2, 4, 4, 32>(q0, q1, num_cus, stream); break;
    case 17: launch_variant<MODE, ROLE, 256, 256, 2, 4, 3, 32>(q0, q1, num_cus, stream); break;
#endif
    default: launch_variant<MODE, ROLE, 128, 256, 2, 4, 3, 64>(q0, q1, num_cus, stream); break;
  }
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
  return (int64_t)(p.n_out + 1) * b_rb <= 0xFFFFFFFFll &&
         (!p.a_rows || (p.a_nrows + 1) * a_rb <= 0xFFFFFFFFll) &&
         (!p.rows_per_group || (int64_t)(p.rows_per_group + 1) * a_rb <= 0xFFFFFFFFll);
}

hipError_t launch_gemm_pair(bool bf16, int op, const GemmProblem& p0, const GemmProblem& p1,
                            int num_cus, hipStream_t stream, int role) {
  const bool any0 = p0.groups > 0 && p0.max_rows > 0, any1 = p1.groups > 0 && p1.max_rows > 0;
  if (!any0 && !any1) return hipSuccess;
  if (bf16 && (!gemm_operands_fit(p0) || !gemm_operands_fit(p1))) return hipErrorInvalidValue;
  if ((any0 ? p0.groups : 0) + (any1 ? p1.groups : 0) > kMaxGroups) return hipErrorInvalidValue;
  if (bf16) {
    GemmProblem q0 = any0 ? p0 : GemmProblem{}, q1 = any1 ? p1 : GemmProblem{};
    auto plain_form = [](const GemmProblem& p) { return !p.k_offsets && !p.lda && !p.ldb && !p.rows_per_group; };
    if (plain_form(q0) && plain_form(q1) &&
        std::max(rows_per_group_bound(q0), rows_per_group_bound(q1)) <= kSkinnyMaxRows) {
#define MOE_SKINNY_DISPATCH(M_)                                            \
  do {                                                                     \
    if (role == 3) launch_skinny<M_, 3>(q0, q1, num_cus, stream);          \
    else if (role == 2) launch_skinny<M_, 2>(q0, q1, num_cus, stream);     \
    else if (role == 1) launch_skinny<M_, 1>(q0, q1, num_cus, stream);     \
    else launch_skinny<M_, 0>(q0, q1, num_cus, stream);                    \
  } while (0)
      if (op == 0) MOE_SKINNY_DISPATCH(kSwiGLU);
      else MOE_SKINNY_DISPATCH(kPlain);
#undef MOE_SKINNY_DISPATCH
      return hipGetLastError();
    }
    const int variant = MOE_GEMM_VARIANT;
#define MOE_GEMM_DISPATCH(M_)                                                  \
  do {                                                                         \
    if (role == 3) launch_shape<M_, 3>(variant, q0, q1, num_cus, stream);      \
    else if (role == 2) launch_shape<M_, 2>(variant, q0, q1, num_cus, stream); \
    else if (role == 1) launch_shape<M_, 1>(variant, q0, q1, num_cus, stream); \
    else launch_shape<M_, 0>(variant, q0, q1, num_cus, stream);                \
  } while (0)
    if (op == 0) MOE_GEMM_DISPATCH(kSwiGLU);
    else MOE_GEMM_DISPATCH(kPlain);
#undef MOE_GEMM_DISPATCH
  } else {
    for (const GemmProblem* p : {&p0, &p1}) {
      if (p->groups == 0 || p->max_rows <= 0) continue;
      const int64_t n = p->max_rows * p->n_out;
      const unsigned grid = (unsigned)((n + 255) / 256);
      const float* A = reinterpret_cast<const float*>(p->a);
      if (op == 0)
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
  return launch_gemm_pair(a.bf16, 1, g2, none, a.num_cus, stream, role);
}

}  // namespace moe
