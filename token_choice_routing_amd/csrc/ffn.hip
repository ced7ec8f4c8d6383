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
//  * Workgroup tile: 128 rows x 128 weight rows x 64 K, four wavefronts of
//    64 x 64. For the gate/up pass the 128 weight rows are 64 gate + 64 up rows
//    of the same output columns, so a lane holds gate and up values of the same
//    (row, column) and applies SwiGLU in registers; h is written once in bf16.
//  * LDS tiles are row-major with 16-byte chunks XOR-swizzled by (row mod 8),
//    so the 32 rows a fragment read touches fall in distinct banks. Two LDS
//    buffers; the next K tile is fetched into registers while the current one
//    feeds the MFMAs, one barrier per K tile.
//  * Persistent grid. Each workgroup builds the tile table from the device
//    offsets (no host round trip for R), and tiles are ordered
//    (expert, column tile, row tile) and cut into 8 contiguous ranges, one per
//    XCD (workgroups are dispatched round-robin over the 8 XCDs), so the row
//    tiles that share one expert's weight panel run on the same L2.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

constexpr int kBM = 128, kBN = 128, kBK = 64, kFfnThreads = 256;
constexpr int kMaxGroups = 320;   // routed groups (<= 256) + the dense shared-expert problem

enum { kSwiGLU = 0, kPlain = 1 };

// element offset of (row, 16-byte chunk) in a [rows][kBK] bf16 LDS tile
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * kBK + ((chunk ^ (row & 7)) << 3);
}

struct TileTable {
  int start[kMaxGroups + 1];
  int len[kMaxGroups + 1];
  int mt[kMaxGroups + 1];
  int nt[kMaxGroups + 1];
  int prefix[kMaxGroups + 1];
};

// Table of (group, column tile, row tile) over problem 0's groups followed by
// problem 1's single dense group. Segment e of a grouped problem is [a, b) with
// a = clamp(offsets[e], 0, max_rows), b = clamp(offsets[e+1], a, max_rows):
// always inside the buffers, exactly the requested segment for valid offsets.
__device__ void build_tile_table(TileTable& tt, const GemmProblem& p0, const GemmProblem& p1,
                                 int oc) {
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    const int G0 = p0.groups, G = p0.groups + p1.groups;
    constexpr int kPer = (kMaxGroups + kWave - 1) / kWave;
    int cnt[kPer], local = 0;
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      const int e = lane * kPer + q;
      int s = 0, l = 0, nt = 0;
      if (e < G) {
        const GemmProblem& pr = e < G0 ? p0 : p1;
        const int ge = e < G0 ? e : e - G0;
        if (pr.offsets) {
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
      const int m = (l + kBM - 1) / kBM;
      if (e <= kMaxGroups) {
        tt.start[e] = s;
        tt.len[e] = l;
        tt.mt[e] = m;
        tt.nt[e] = nt;
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

// MODE kSwiGLU writes h as bf16 (the next MFMA's input); kPlain writes float32.
// ROLE only names the launch in profiles (the code is identical): 0 standalone
// grouped, 1 standalone single segment, 2 the layer's routed + shared launch.
template <int MODE, int ROLE>
__global__ void __launch_bounds__(kFfnThreads)
grouped_gemm_bf16_kernel(GemmProblem p0, GemmProblem p1) {
  __shared__ TileTable tt;
  __shared__ __attribute__((aligned(16))) bf16_t smem[2][2][kBM * kBK];  // [buf][A|B][tile]
  constexpr int OC = MODE == kSwiGLU ? kBN / 2 : kBN;  // output columns per tile
  build_tile_table(tt, p0, p1, OC);
  const int G0 = p0.groups, G = p0.groups + p1.groups;
  const int total = tt.prefix[kMaxGroups];

  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int wm = wave & 1, wn = wave >> 1;
  const int half = lane >> 5, l32 = lane & 31;
  const int ld_chunk = tid & 7, ld_row = tid >> 3;  // + 32 * i

  // XCD-contiguous tile ranges
  const int P = gridDim.x;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int per_xcd_blocks = P >> 3;
  const int S = (total + 7) / 8;
  const int r_begin = xcd * S, r_end = min(total, r_begin + S);

  for (int L = r_begin + slot; L < r_end; L += per_xcd_blocks) {
    // locate (group, column tile, row tile)
    int lo = 0, hi = G;  // prefix[lo] <= L < prefix[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (tt.prefix[mid] <= L) lo = mid; else hi = mid;
    }
    const int e = lo;
    const bool second = e >= G0;
    const GemmProblem& pr = second ? p1 : p0;
    const int ge = second ? e - G0 : e;
    const int Nout = pr.n_out, Kdim = pr.k_dim;
    const int nk = (Kdim + kBK - 1) / kBK;
    const int local = L - tt.prefix[e];
    const int mt = tt.mt[e];
    const int ntile = local / mt, mtile = local - ntile * mt;
    const int m0 = tt.start[e] + mtile * kBM;
    const int rows_valid = min(kBM, tt.start[e] + tt.len[e] - m0);

    // global sources of this thread's 4 A rows and 4 B rows: always a valid row
    // (clamped). Rows past the segment and columns past n_out only produce outputs
    // that are never stored, so their loads need no masking; columns past k_dim
    // (last K tile only) are zeroed at stash. No branch or select sits between a
    // load and the MFMAs, so all eight loads of the next tile stay in flight.
    const bf16_t* asrc[4];
    const bf16_t* bsrc[4];
    int64_t arow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = ld_row + 32 * i;
      arow[i] = m0 + (r < rows_valid ? r : 0);
    }
    if (pr.a_rows) {
      int32_t src_row[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) src_row[i] = pr.a_rows[arow[i]];
#pragma unroll
      for (int i = 0; i < 4; ++i) arow[i] = min<int64_t>(max<int64_t>(src_row[i], 0), pr.a_nrows - 1);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = ld_row + 32 * i;
      asrc[i] = pr.a + arow[i] * Kdim;
      int n;
      const bf16_t* base;
      if (MODE == kSwiGLU) {
        n = ntile * OC + (r & (OC - 1));
        base = r < OC ? pr.b0 : pr.b1;
      } else {
        n = ntile * OC + r;
        base = pr.b0;
      }
      bsrc[i] = base + ((int64_t)ge * Nout + (n < Nout ? n : 0)) * Kdim;
    }
    u32x4_t ra[4], rb[4];
    auto fetch = [&](int kt) {
      const int k = kt * kBK + ld_chunk * 8;
      const int kc = k < Kdim ? k : 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ra[i] = *reinterpret_cast<const u32x4_t*>(asrc[i] + kc);
        rb[i] = *reinterpret_cast<const u32x4_t*>(bsrc[i] + kc);
      }
    };
    auto stash = [&](int buf, int kt) {
      if ((kt + 1) * kBK > Kdim && kt * kBK + ld_chunk * 8 >= Kdim) {  // K tail only
#pragma unroll
        for (int i = 0; i < 4; ++i) ra[i] = rb[i] = u32x4_t{0, 0, 0, 0};
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = ld_row + 32 * i;
        *reinterpret_cast<u32x4_t*>(&smem[buf][0][lds_off(r, ld_chunk)]) = ra[i];
        *reinterpret_cast<u32x4_t*>(&smem[buf][1][lds_off(r, ld_chunk)]) = rb[i];
      }
    };

    f32x16_t acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b) acc[a][b] = f32x16_t{};

    fetch(0);
    stash(0, 0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int buf = kt & 1;
      if (kt + 1 < nk) fetch(kt + 1);
      const bf16_t* As = smem[buf][0];
      const bf16_t* Bs = smem[buf][1];
#pragma unroll
      for (int ks = 0; ks < kBK / 16; ++ks) {
        const int ch = ks * 2 + half;
        bf16x8_t wf[2], af[2];
#pragma unroll
        for (int ns = 0; ns < 2; ++ns) {
          const int brow = MODE == kSwiGLU ? ns * OC + wn * 32 + l32 : wn * 64 + ns * 32 + l32;
          wf[ns] = *reinterpret_cast<const bf16x8_t*>(&Bs[lds_off(brow, ch)]);
        }
#pragma unroll
        for (int ms = 0; ms < 2; ++ms) {
          const int arow = wm * 64 + ms * 32 + l32;
          af[ms] = *reinterpret_cast<const bf16x8_t*>(&As[lds_off(arow, ch)]);
        }
#pragma unroll
        for (int ns = 0; ns < 2; ++ns)
#pragma unroll
          for (int ms = 0; ms < 2; ++ms)
            acc[ns][ms] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[ns], af[ms], acc[ns][ms], 0, 0, 0);
      }
      if (kt + 1 < nk) stash(buf ^ 1, kt + 1);
      __syncthreads();
    }

    // epilogue: lane owns row (l32) of each 32-row subtile, 4 consecutive columns per group
#pragma unroll
    for (int ms = 0; ms < 2; ++ms) {
      const int rl = wm * 64 + ms * 32 + l32;
      if (rl >= rows_valid) continue;
      if (MODE == kSwiGLU) {
        bf16_t* crow = static_cast<bf16_t*>(pr.out) + (int64_t)(m0 + rl) * Nout;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = ntile * OC + wn * 32 + 8 * g + 4 * half;
          if (col < Nout) {
            float h[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) h[j] = silu(acc[0][ms][4 * g + j]) * acc[1][ms][4 * g + j];
            *reinterpret_cast<u32x2_t*>(crow + col) = u32x2_t{pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3])};
          }
        }
      } else {
        float* crow = static_cast<float*>(pr.out) + (int64_t)(m0 + rl) * Nout;
#pragma unroll
        for (int ns = 0; ns < 2; ++ns)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int col = ntile * OC + wn * 64 + ns * 32 + 8 * g + 4 * half;
            if (col < Nout) {
              const f32x16_t& v = acc[ns][ms];
              *reinterpret_cast<f32x4_t*>(crow + col) =
                  f32x4_t{v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]};
            }
          }
      }
    }
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

static unsigned gemm_grid(const GemmProblem& p0, const GemmProblem& p1, int oc, int num_cus) {
  auto upper = [&](const GemmProblem& p) -> int64_t {
    if (p.groups == 0 || p.max_rows <= 0) return 0;
    return (p.max_rows / kBM + p.groups) * ((p.n_out + oc - 1) / oc);
  };
  const int64_t tiles = upper(p0) + upper(p1);
  // persistent grid: 2 workgroups per CU (about 68 KiB LDS each), a multiple of 8
  const int cap = std::max(8, num_cus * 2 / 8 * 8);
  return (unsigned)std::max<int64_t>(8, std::min<int64_t>(cap, (tiles + 7) / 8 * 8));
}

hipError_t launch_gemm_pair(bool bf16, int op, const GemmProblem& p0, const GemmProblem& p1,
                            int num_cus, hipStream_t stream, int role) {
  const bool any0 = p0.groups > 0 && p0.max_rows > 0, any1 = p1.groups > 0 && p1.max_rows > 0;
  if (!any0 && !any1) return hipSuccess;
  if (bf16) {
    const int oc = op == 0 ? kBN / 2 : kBN;
    GemmProblem q0 = any0 ? p0 : GemmProblem{}, q1 = any1 ? p1 : GemmProblem{};
    const unsigned grid = gemm_grid(q0, q1, oc, num_cus);
#define MOE_GEMM_LAUNCH(M_, R_) grouped_gemm_bf16_kernel<M_, R_><<<grid, kFfnThreads, 0, stream>>>(q0, q1)
    if (op == 0) {
      if (role == 2) MOE_GEMM_LAUNCH(kSwiGLU, 2);
      else if (role == 1) MOE_GEMM_LAUNCH(kSwiGLU, 1);
      else MOE_GEMM_LAUNCH(kSwiGLU, 0);
    } else {
      if (role == 2) MOE_GEMM_LAUNCH(kPlain, 2);
      else if (role == 1) MOE_GEMM_LAUNCH(kPlain, 1);
      else MOE_GEMM_LAUNCH(kPlain, 0);
    }
#undef MOE_GEMM_LAUNCH
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
