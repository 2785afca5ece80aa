// CoWindow Attention forward, bf16 in/out, head dim 128, for gfx950.
//
// One work item = (KV head h, q-block of Bq = 256 / G tokens): the query rows of the G
// query heads that share KV head h (slinene.github.io ai-papers-daily page, method key
// point 3: windows follow the KV head, so one K/V tile read from HBM serves all G query
// heads).  Rows are token-major (row r = token * G + head-in-group), so the item's Q is
// one strided run of G * 256 bytes per token.  Four waves own 64 rows each, as two
// 32-column blocks of v_mfma_f32_32x32x16_bf16.
//
// The item walks the planner's row list of visible 64-key blocks (masked blocks are
// never touched).  Per block t, in one pipelined loop iteration:
//   [A] S(t+1)^T = K(t+1) Q^T on MFMA: K (A operand, one key row per lane) and Q^T (B
//       operand) from LDS, so each lane owns one query row (column) and 16 of every 32
//       keys; a boundary (PARTIAL) block gets the window predicate per element at the
//       start of its own iteration;
//   [B] online softmax of S(t) in base 2 (scale * log2 e folded into one FMA), the row
//       max taken across the two lane halves of a column; the running max only moves
//       when a row's tile max exceeds it by more than 8 (log2 units) — exact, because
//       O / l does not depend on the reference, and P stays <= 256; P(t) is computed
//       with the current reference and recomputed only on such a (rare) move;
//   [C] O^T += V(t)^T P(t)^T: P^T goes from the C-layout accumulator straight into the B
//       operand (no LDS round trip) and V^T is read from the row-major LDS tile with
//       ds_read_b64_tr_b16, two 4-key runs per operand matching the accumulator layout.
// [A] has no dependence on [B], so the scheduler overlaps the two (MFMA and VALU run
// in parallel within a wave).
//
// Memory pipeline: K and V are double-buffered in LDS and filled by direct
// global->LDS loads (global_load_lds_dwordx4, no staging registers); the loads of K(t+2)
// and V(t+1) are issued right after the single barrier of iteration t and waited for at
// the next one.  LDS rows are 256 bytes with the 16-byte chunks XOR-swizzled by a function
// of the row, so both the row-wise operand reads and the transposed V reads are free of
// bank conflicts.
// Output: O / l in bf16 and LSE = ln 2 * (m + log2 l) in fp32.
//
// MFMA lane layouts of v_mfma_f32_32x32x16_bf16 (n = lane % 32, h2 = lane / 32):
//   A (32 x 16): A[n][8 h2 + e]   B (16 x 32): B[8 h2 + e][n]
//   C (32 x 32): element i of 16 is C[8 (i / 4) + 4 h2 + i % 4][n]

#include "device_common.h"

namespace cowa {
namespace {

constexpr int D = 128;
constexpr int WAVES = 4;
constexpr int ROWS = kFwdRows;       // 256 rows per item
constexpr int WROWS = ROWS / WAVES;  // 64 rows per wave
constexpr int CB = WROWS / 32;       // 2 column blocks of 32 per wave
constexpr int BK = kFwdBk;           // 64 keys per tile
constexpr int KB2 = BK / 32;         // 2 key blocks of 32
constexpr int TILE = BK * D;         // elements per K or V tile
constexpr float kRescaleThreshold = 8.0f;

// LDS tiles: 256-byte rows with XOR-swizzled 16-byte chunks (lds_sw / lds_swz).
__device__ __forceinline__ int sw(int r) { return lds_sw(r); }
__device__ __forceinline__ int swz(int r, int e) { return lds_swz(r, e); }

// x * alpha for a value held in an accumulation register, done in place: read to a VGPR,
// multiply, write back.  Only used on the rare rescale path, long after the MFMA that
// last wrote the register (a whole tile of LDS reads and MFMAs lies in between).
__device__ __forceinline__ float agpr_scale(float x, float alpha) {
  float t;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(t) : "a"(x));
  t *= alpha;
  float r;
  asm volatile("v_accvgpr_write_b32 %0, %1" : "=a"(r) : "v"(t));
  return r;
}

__global__ __launch_bounds__(256, 1) void fwd_bf16_d128_kernel(FwdArgs a) {
  __shared__ __attribute__((aligned(1024))) __bf16 sQ[ROWS * D];
  __shared__ __attribute__((aligned(1024))) __bf16 sK[2 * TILE];
  __shared__ __attribute__((aligned(1024))) __bf16 sV[2 * TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 31;
  const int h2 = lane >> 5;
  const int item = a.row_order[blockIdx.x];
  const int b = blockIdx.y;
  const int h = item / a.nqb;
  const int qb = item - h * a.nqb;
  const int G = a.G;
  const int Bq = a.Bq;
  const int off = a.Lk - a.Lq;
  const HeadBand band = head_band(a.win, h);

  const __bf16* Q = (const __bf16*)a.q;
  const __bf16* K = (const __bf16*)a.k;
  const __bf16* V = (const __bf16*)a.v;

  int tok[CB], hq[CB];
  bool rvalid[CB];
#pragma unroll
  for (int c = 0; c < CB; ++c) {
    const int r = wave * WROWS + c * 32 + n;
    const int rt = r / G;
    tok[c] = qb * Bq + rt;
    hq[c] = h * G + (r - rt * G);
    rvalid[c] = (rt < Bq) && (tok[c] < a.Lq);
  }

  // ---- direct loads.  Lane L of a 1 KB copy fills row r = 4 * blk + L / 16, physical
  // chunk L % 16, so it fetches logical chunk (L % 16) ^ sw(r) of that row.
  const int lrow = lane >> 4;
  const int lchunk = lane & 15;
  {  // this wave's 64 query rows (rows past the q-block or Lq read a valid row; unused)
    __bf16* dst = sQ + wave * WROWS * D;
#pragma unroll
    for (int u = 0; u < WROWS / 4; ++u) {
      const int r = wave * WROWS + 4 * u + lrow;
      const int rt = r / G;
      int t = qb * Bq + rt;
      int g = r - rt * G;
      if (rt >= Bq || t >= a.Lq) {
        t = min(qb * Bq, a.Lq - 1);
        g = 0;
      }
      const int c = lchunk ^ sw(r);
      g2lds(Q + (((int64_t)b * a.Lq + t) * a.Hq + h * G + g) * D + 8 * c, dst + 4 * u * D);
    }
  }
  auto load_tile = [&](const __bf16* src, __bf16* dst, int kb) {
    // wave w copies rows 16 w .. 16 w + 15 (keys past Lk read key Lk - 1; masked)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = 16 * wave + 4 * u + lrow;
      const int j = min(kb * BK + r, a.Lk - 1);
      const int c = lchunk ^ sw(r);
      g2lds(src + (((int64_t)b * a.Lk + j) * a.Hkv + h) * D + 8 * c, dst + (16 * wave + 4 * u) * D);
    }
  };

  f32x16 acc[CB][4];
#pragma unroll
  for (int c = 0; c < CB; ++c)
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[c][db][i] = 0.f;
  float m[CB], l[CB];
#pragma unroll
  for (int c = 0; c < CB; ++c) {
    m[c] = -INFINITY;
    l[c] = 0.f;
  }

  const int e0 = a.row_ptr[item];
  const int nt = a.row_ptr[item + 1] - e0;
  const __bf16* sQw = sQ + wave * WROWS * D;

  // tr-read addressing for the V^T operand: 16-lane group gg covers d columns
  // 16 (gg & 1) .. +15 of a 32-column block and key run 4 (gg >> 1) (+8)
  const int gg = lane >> 4, j16 = lane & 15;
  const int vrow = 4 * (gg >> 1) + (j16 >> 2);
  const int vcol = 16 * (gg & 1) + 4 * (j16 & 3);

  // boundary tile t: branch-free window predicate per element
  auto mask = [&](f32x16 (&s)[KB2][CB], int ent) {
    if (ent & 1) {
      const int kb = ent >> 1;
#pragma unroll
      for (int c = 0; c < CB; ++c) {
        const int p = tok[c] + off;
#pragma unroll
        for (int k2 = 0; k2 < KB2; ++k2)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int j = kb * BK + 32 * k2 + 8 * (i >> 2) + 4 * h2 + (i & 3);
            const bool vis = rvalid[c] & visible(p, j, a.Lk, a.win.sink, a.win.near_w, band);
            s[k2][c][i] = vis ? s[k2][c][i] : -INFINITY;
          }
      }
    }
  };

  auto scores = [&](f32x16 (&s)[KB2][CB], int t) {
    const __bf16* kt = sK + (t & 1) * TILE;
#pragma unroll
    for (int k2 = 0; k2 < KB2; ++k2)
#pragma unroll
      for (int c = 0; c < CB; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[k2][c][i] = 0.f;
#pragma unroll
    for (int dd = 0; dd < D / 16; ++dd) {
      bf16x8 qf[CB];
#pragma unroll
      for (int c = 0; c < CB; ++c) qf[c] = load16(sQw + swz(c * 32 + n, 16 * dd + 8 * h2));
#pragma unroll
      for (int k2 = 0; k2 < KB2; ++k2) {
        const bf16x8 kf = load16(kt + swz(32 * k2 + n, 16 * dd + 8 * h2));
#pragma unroll
        for (int c = 0; c < CB; ++c) s[k2][c] = mfma32x32x16(kf, qf[c], s[k2][c]);
      }
    }
  };

  // List entries of tiles t .. t+2 are kept in registers and entry t+3 is loaded one
  // iteration ahead: a load of it issued after the direct copies and waited for at once
  // would also wait for those copies (one in-order counter covers both).
  int ent0 = 0, ent1 = 0, ent2 = 0;
  auto iteration = [&](int t, f32x16 (&cur)[KB2][CB], f32x16 (&next)[KB2][CB]) {
    wait_loads_and_barrier();  // K(t+1), V(t), entry t+3 resident; every wave is done with t-1
    const int ent3 = (t + 3 < nt) ? a.row_ent[e0 + t + 3] : 0;  // made uniform when used
    if (t + 2 < nt) load_tile(K, sK + (t & 1) * TILE, __builtin_amdgcn_readfirstlane(ent2) >> 1);
    if (t + 1 < nt) load_tile(V, sV + ((t + 1) & 1) * TILE, __builtin_amdgcn_readfirstlane(ent1) >> 1);
    mask(cur, __builtin_amdgcn_readfirstlane(ent0));
    ent0 = ent1;
    ent1 = ent2;
    ent2 = ent3;

    // Interleaved block: step i issues one MFMA of S(t+1) (dd = i / 4, (k2, c) = i % 4;
    // past the last tile it reads a resident buffer and the result is unused), then the
    // softmax work of two elements of S(t): exp2 with the current reference, running max,
    // and every 4 steps the bf16 packing and row sum of 8 probabilities.  The scheduling
    // fences keep this order, so the matrix core and the VALU run at the same time.
    const __bf16* kt = sK + ((t + 1) & 1) * TILE;
#pragma unroll
    for (int k2 = 0; k2 < KB2; ++k2)
#pragma unroll
      for (int c = 0; c < CB; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) next[k2][c][i] = 0.f;
    bf16x8 kf[2][KB2], qf[2][CB];
#pragma unroll
    for (int x = 0; x < KB2; ++x) kf[0][x] = load16(kt + swz(32 * x + n, 8 * h2));
#pragma unroll
    for (int x = 0; x < CB; ++x) qf[0][x] = load16(sQw + swz(32 * x + n, 8 * h2));
    float ref[CB], mx[CB], sum[CB];
#pragma unroll
    for (int c = 0; c < CB; ++c) {
      ref[c] = (m[c] == -INFINITY) ? 0.f : m[c];
      mx[c] = -INFINITY;
      sum[c] = 0.f;
    }
    bf16x8 pf[KB2][CB][2];
    float pb[8];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int dd = i >> 2, k2 = (i >> 1) & 1, c = i & 1;
      if ((i & 3) == 0 && dd + 1 < D / 16) {
#pragma unroll
        for (int x = 0; x < KB2; ++x) kf[(dd + 1) & 1][x] = load16(kt + swz(32 * x + n, 16 * (dd + 1) + 8 * h2));
#pragma unroll
        for (int x = 0; x < CB; ++x) qf[(dd + 1) & 1][x] = load16(sQw + swz(32 * x + n, 16 * (dd + 1) + 8 * h2));
      }
      next[k2][c] = mfma32x32x16(kf[dd & 1][k2], qf[dd & 1][c], next[k2][c]);
      __builtin_amdgcn_sched_barrier(0);
      // elements 2i, 2i+1 of S(t) in (c, k2, hf, e2) order
      const int ec = i >> 4, ek2 = (i >> 3) & 1, ehf = (i >> 2) & 1, e2 = 2 * (i & 3);
      const float x0 = cur[ek2][ec][8 * ehf + e2], x1 = cur[ek2][ec][8 * ehf + e2 + 1];
      mx[ec] = fmaxf(mx[ec], fmaxf(x0, x1));
      pb[e2] = __builtin_amdgcn_exp2f(fmaf(x0, a.scale_log2, -ref[ec]));
      pb[e2 + 1] = __builtin_amdgcn_exp2f(fmaf(x1, a.scale_log2, -ref[ec]));
      sum[ec] += pb[e2] + pb[e2 + 1];  // fp32 row sum (it sets LSE, which the backward reuses)
      if ((i & 3) == 3)
        pf[ek2][ec][ehf] = join(to_bf16x4(pb[0], pb[1], pb[2], pb[3]), to_bf16x4(pb[4], pb[5], pb[6], pb[7]));
      __builtin_amdgcn_sched_barrier(0);
    }

    float mt[CB];
    bool need[CB];
#pragma unroll
    for (int c = 0; c < CB; ++c) {
      const float x = fmaxf(mx[c], __shfl_xor(mx[c], 32));
      mt[c] = x * a.scale_log2;
      need[c] = mt[c] > m[c] + kRescaleThreshold;
    }
    if (__builtin_amdgcn_ballot_w64(need[0] | need[1]) != 0) {
      // rare: rows whose max moved past the threshold take it as their new reference;
      // their accumulators, sums and P(t) are rescaled / recomputed, the other rows keep
      // theirs
#pragma unroll
      for (int c = 0; c < CB; ++c) {
        const float mn = need[c] ? mt[c] : m[c];
        const float alpha = (m[c] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m[c] - mn);
        m[c] = mn;
        l[c] *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[c][db][i] = agpr_scale(acc[c][db][i], alpha);
      }
#pragma unroll
      for (int c = 0; c < CB; ++c) {
        const float rf = (m[c] == -INFINITY) ? 0.f : m[c];
        float s2 = 0.f;
#pragma unroll
        for (int k2 = 0; k2 < KB2; ++k2)
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            float p[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
              p[e] = __builtin_amdgcn_exp2f(fmaf(cur[k2][c][8 * hf + e], a.scale_log2, -rf));
#pragma unroll
            for (int e = 0; e < 8; ++e) s2 += p[e];
            const bf16x8 pn = join(to_bf16x4(p[0], p[1], p[2], p[3]), to_bf16x4(p[4], p[5], p[6], p[7]));
            pf[k2][c][hf] = need[c] ? pn : pf[k2][c][hf];
          }
        sum[c] = need[c] ? s2 : sum[c];
      }
    }
#pragma unroll
    for (int c = 0; c < CB; ++c) l[c] += sum[c];
    // O^T += V(t)^T P(t)^T
    // (k2, hf) outermost so that the 8 accumulators rotate: each one is next updated only
    // after 7 independent MFMAs
    const __bf16* vt = sV + (t & 1) * TILE;
#pragma unroll
    for (int k2 = 0; k2 < KB2; ++k2) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const int r0 = 32 * k2 + 16 * hf + vrow;
          const int col = 32 * db + vcol;
          const bf16x8 vf = join(lds_read_tr4(vt + swz(r0, col)), lds_read_tr4(vt + swz(r0 + 8, col)));
#pragma unroll
          for (int c = 0; c < CB; ++c) acc[c][db] = mfma32x32x16(vf, pf[k2][c][hf], acc[c][db]);
        }
      }
    }
  };

  if (nt > 0) {
    ent0 = a.row_ent[e0];
    ent1 = nt > 1 ? a.row_ent[e0 + 1] : 0;
    ent2 = nt > 2 ? a.row_ent[e0 + 2] : 0;
    load_tile(K, sK, __builtin_amdgcn_readfirstlane(ent0) >> 1);
    load_tile(V, sV, __builtin_amdgcn_readfirstlane(ent0) >> 1);
    if (nt > 1) load_tile(K, sK + TILE, __builtin_amdgcn_readfirstlane(ent1) >> 1);
    f32x16 sa[KB2][CB], sb[KB2][CB];
    wait_loads_and_barrier();
    scores(sa, 0);
    for (int t = 0; t < nt; t += 2) {
      iteration(t, sa, sb);
      if (t + 1 < nt) iteration(t + 1, sb, sa);
    }
  }

  // ---- finalize: l summed over the two lane halves of a column
  __bf16* O = (__bf16*)a.o;
#pragma unroll
  for (int c = 0; c < CB; ++c) {
    float lt = l[c] + __shfl_xor(l[c], 32);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    if (rvalid[c]) {
      __bf16* op = O + (((int64_t)b * a.Lq + tok[c]) * a.Hq + hq[c]) * D + 4 * h2;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const bf16x4 v = to_bf16x4(acc[c][db][4 * q4] * inv, acc[c][db][4 * q4 + 1] * inv,
                                     acc[c][db][4 * q4 + 2] * inv, acc[c][db][4 * q4 + 3] * inv);
          *(u32x2*)(op + 32 * db + 8 * q4) = __builtin_bit_cast(u32x2, v);
        }
      if (h2 == 0)
        a.lse[((int64_t)b * a.Hq + hq[c]) * a.Lq + tok[c]] =
            lt > 0.f ? (m[c] + log2f(lt)) * kLn2 : -INFINITY;
    }
  }
}

}  // namespace

hipError_t launch_fwd_bf16_d128(const FwdArgs& a, hipStream_t s) {
  dim3 grid(a.n_items, a.B);
  hipLaunchKernelGGL(fwd_bf16_d128_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace cowa
