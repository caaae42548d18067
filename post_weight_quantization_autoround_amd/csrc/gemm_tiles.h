// MFMA GEMM tiles of the tuning loop (gfx950), shared by the library's
// launchers.  See gemm_kernels.hip for the operand mapping of the two GEMMs.
//
// C[i, j] = sum_r A[i, r] * B[j, r]; both operands are read along the
// reduction index r in 16-byte chunks.  A workgroup computes a BM x BN tile
// with NWM x NWN wavefronts, each owning a (BM/NWM) x (BN/NWN) sub-tile of
// 32 x 32 MFMA blocks with fp32 accumulators.  Operand tiles of BK
// reduction elements are staged through LDS, double buffered with one
// barrier per BK step: the global loads of step k+1 are issued before the
// MFMAs of step k, and the fragments of sub-step s+1 are read from LDS while
// the MFMAs of sub-step s run.  LDS rows are padded by 16 bytes so the
// fragment reads of 32 consecutive rows hit distinct banks.  Interior tiles
// take an unmasked load path; edge tiles mask rows and reduction columns.
#pragma once

#include <type_traits>

#include "ar_internal.h"

namespace ar {
namespace gemm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;
typedef const __attribute__((address_space(1))) void gbl_void;
typedef short lds_v4s_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) lds_v4s_t lds_v4s;

// Workgroup barrier without the release/acquire fences of __syncthreads():
// those wait for every outstanding global load, which would drain the DMA
// pipeline.  Callers wait for their own LDS-bound loads first (wait_vmcnt).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    // s_waitcnt vmcnt(N); a compiler barrier too, so no memory access is
    // moved across it
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// f(std::integral_constant<int, i>) for i = 0 .. N-1, unrolled at compile time.
template <int N, typename F, int I = 0>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<N, F, I + 1>(static_cast<F&&>(f));
    }
}


struct SchedView {
    const int32_t* ids;  // NULL: identity
    __device__ __forceinline__ int64_t id(int64_t s) const { return ids ? (int64_t)ids[s] : s; }
};

// Step indices of a launch: the schedule row of its minibatch and, for the
// fused update, the parameter buffers it reads (src) and writes (dst) and
// the step whose learning rate applies.  Taken from the state after (or,
// for the forward GEMM, before) the step's loss decision.
struct StepView {
    int32_t row, src, dst, t;
};
__device__ __forceinline__ StepView step_view(const GemmArgs& a) {
    StepView v{0, 0, 0, 0};
    if (a.state) {
        v.row = a.after_decide ? a.state->t_eval : a.state->step;
        v.src = a.state->src;
        v.dst = a.state->dst;
        v.t = a.state->t_eval;
    }
    return v;
}

// The step's loss decision taken inside the fused weight-gradient launch
// (GemmArgs::dec_partials), in three parts:
//  - fold_begin, at the start: the schedule row is the step the forward GEMM
//    evaluated (the state is not committed yet), and each lane loads up to
//    four loss partials so their latency hides behind the main loop;
//  - fold_decide, before the epilogue: every wavefront sums the partials in
//    the fixed order of wave_loss_sum and decides on the uncommitted state;
//  - fold_arrive, at the end: the workgroup counts its arrival, and the last
//    one to arrive commits the decision and clears the counter.  Every
//    workgroup has read the state before it arrives, so none reads a
//    committed state.
// PRE partials per lane are loaded at the start (0: at the decision; the
// kernels whose main loop needs every register).
template <int PRE>
struct FoldPre {
    double p[PRE > 0 ? PRE : 1];
};
template <int PRE>
__device__ __forceinline__ bool fold_begin(const GemmArgs& a, StepView& v, FoldPre<PRE>& pre) {
    const StepState* st = a.dec_state;
    if (st->halted) return false;      // stopped earlier: no arrival, nothing to commit
    v.row = st->step;
    const int lane = (int)__lane_id();
#pragma unroll
    for (int j = 0; j < PRE; ++j) pre.p[j] = (lane + 64 * j < a.dec_np) ? a.dec_partials[lane + 64 * j] : 0.0;
    return true;
}
template <int PRE>
__device__ __forceinline__ double fold_decide(const GemmArgs& a, StepView& v, const FoldPre<PRE>& pre) {
    const int lane = (int)__lane_id();
    double acc = 0.0;                  // the order of wave_loss_sum
#pragma unroll
    for (int j = 0; j < PRE; ++j)
        if (lane + 64 * j < a.dec_np) acc += pre.p[j];
    for (int i = lane + 64 * PRE; i < a.dec_np; i += 64) acc += a.dec_partials[i];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    // every lane holds the same sum: keep it (and what follows) in scalar registers
    const uint64_t bits = __builtin_bit_cast(uint64_t, acc);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)bits);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(bits >> 32));
    const double L = __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo) * a.dec_inv;
    const StepState* st = a.dec_state;
    const int32_t cur = st->cur;
    v.t = v.row;
    v.src = cur;
    v.dst = (__builtin_isfinite(L) && L < st->best_loss) ? 1 - cur : cur;
    return L;
}
__device__ __forceinline__ void fold_arrive(const GemmArgs& a, double L) {
    if (threadIdx.x == 0 && atomicAdd(a.dec_arrivals, 1) == (int)gridDim.x - 1) {
        commit_decision(a.dec_state, a.dec_trace, a.dec_iters, L);
        atomicExch(a.dec_arrivals, 0);
    }
}

__device__ __forceinline__ SchedView sched_view(const GemmArgs& a, int32_t row) {
    SchedView v;
    v.ids = a.sched ? a.sched + (int64_t)row * a.nseg : nullptr;
    return v;
}

// Element offset of row i of an operand (column part added separately).
__device__ __forceinline__ int64_t row_offset(const Operand& op, const SchedView& sv, int64_t i) {
    if (op.seg_len > 0 && !op.seg_cols) {
        const int64_t seg = i / op.seg_len;
        return sv.id(seg) * op.seg_stride + (i - seg * op.seg_len) * op.ld;
    }
    return i * op.ld;
}

// Element offset of reduction column k0, the start of a BK tile (a tile
// never crosses a segment: BK divides the segment length).
__device__ __forceinline__ int64_t col_offset(const Operand& op, const SchedView& sv, int64_t k0) {
    if (op.seg_len > 0 && op.seg_cols) {
        const int64_t seg = k0 / op.seg_len;
        return sv.id(seg) * op.seg_stride + (k0 - seg * op.seg_len);
    }
    return k0;
}

// Tile of workgroup blockIdx.x.  Workgroups are dispatched to the 8 XCDs in
// turn (workgroup b runs on XCD b % 8) and each XCD has its own L2, so the
// tile grid is cut into 8 rectangles of tm x tn tiles, one per XCD, with the
// split (a x 8/a) that minimises the operand rows each XCD must pull into
// its L2 (tm*BM + tn*BN); within an XCD tiles run in bands (below).  Grids
// that do not split evenly fall back to row-major order.
template <int BM, int BN>
__device__ __forceinline__ void tile_coords(int64_t tiles_m, int64_t tiles_n, int64_t& tile_m, int64_t& tile_n) {
    const int64_t b = blockIdx.x;
    int best_a = 0;
    int64_t best_cost = 0;
#pragma unroll
    for (int a = 1; a <= 8; a <<= 1) {
        if (tiles_m % a != 0 || tiles_n % (8 / a) != 0) continue;
        const int64_t cost = (tiles_m / a) * BM + (tiles_n / (8 / a)) * BN;
        if (best_a == 0 || cost < best_cost) {
            best_a = a;
            best_cost = cost;
        }
    }
    if (best_a == 0) {
        tile_m = b % tiles_m;
        tile_n = b / tiles_m;
        return;
    }
    const int64_t rm = tiles_m / best_a, rn = tiles_n / (8 / best_a);
    const int64_t xcd = b & 7, local = b >> 3;
    const int64_t ra = xcd / (8 / best_a), rb = xcd % (8 / best_a);
    // Rectangles of more than one round (32 CUs per XCD) are walked in bands
    // of up to 4 tile rows, column by column (the rows left over form a last,
    // shorter band): the ~32 tiles an XCD runs at once span 4 A row blocks
    // and 8 B column blocks instead of one tall column of A blocks.  A single
    // round runs column by column.
    const int64_t hb = (rm * rn <= 32 || rm < 4) ? rm : 4;
    const int64_t full = (rm / hb) * hb * rn;
    if (local < full) {
        const int64_t band = local / (hb * rn), w = local % (hb * rn);
        tile_m = ra * rm + band * hb + w % hb;
        tile_n = rb * rn + w / hb;
    } else {
        const int64_t rest = rm - (rm / hb) * hb, w = local - full;
        tile_m = ra * rm + (rm / hb) * hb + w % rest;
        tile_n = rb * rn + w / rest;
    }
}

// Epilogue over one wavefront's accumulators.  Accumulator r of the 32 x 32
// block (tm, tn) holds row 8*(r/4) + 4*(lane/32) + r%4, column lane%32, so a
// half-wavefront covers 32 consecutive columns of one row: stores and the
// reference reads are contiguous along j.
//   EPI_STORE: out[i, j] = C.
//   EPI_LOSS : rows are output features n, columns the minibatch tokens m
//              (segmented by sample); D = C - Yref[sample, n, token] (D = C
//              when yref is NULL: the A operand was already w^ - W),
//              partial sum of D^2, dY^T[n, m] = dscale * D.
template <int TM, int TN, int EPI>
__device__ __forceinline__ void epilogue(const GemmArgs& a, const SchedView& sv, floatx16 (&acc)[TM][TN],
                                         int64_t row0, int64_t col0, int lane, double* red) {
    const int half = lane >> 5;
    const int cl = lane & 31;
    float lsum = 0.0f;
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
        const int64_t j = col0 + tn * 32 + cl;
        const bool jok = j < a.J;
        int64_t pj = 0;   // reference offset of column j (sample block + token)
        if (EPI == EPI_LOSS && jok) {
            const int64_t seg = j / a.yref_T;
            pj = sv.id(seg) * a.yref_seg_stride + (j - seg * a.yref_T);
        }
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t i = row0 + tm * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
                if (!jok || i >= a.I) continue;
                if (EPI == EPI_STORE) {
                    a.out[i * a.ldc + j] = acc[tm][tn][r];
                } else {
                    const float d = a.yref ? acc[tm][tn][r] - a.yref[i * a.yref_ld + pj] : acc[tm][tn][r];
                    lsum += d * d;
                    if (a.dyt_bf16)
                        static_cast<uint16_t*>(a.dyt)[i * a.lddyt + j] = f32_to_bf16(a.dscale * d);
                    else
                        static_cast<float*>(a.dyt)[i * a.lddyt + j] = a.dscale * d;
                }
            }
        }
    }
    if (EPI == EPI_LOSS) {
        double v = (double)lsum;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
        if (lane == 0) red[threadIdx.x >> 6] = v;
    }
}

// Fused wgrad epilogue (EPI_STE): the accumulators hold G = dL/dw^ for rows
// n (weight rows) and columns k of whole groups.  The tile is staged through
// the LDS the main loop no longer needs, RPP rows at a time, and re-read
// row-major so each thread owns 8 consecutive weights and the g/8 lanes of a
// group are adjacent.  Per weight: straight-through gradient dV = G s m and
// the group terms (AutoRound blog sec. 3: rounding passed through as the
// identity), SignSGD move of V; per group (segmented lane reduction):
// dalpha = mx/Q sum G c, dbeta = mn sum G ((1 - m) - c/Q) and their SignSGD
// moves; finally the updated state is fake-quantized to bf16 for the next
// step's forward GEMM.  Reads W and V, writes V, alpha, beta and w^: G never
// leaves the chip.
__device__ __forceinline__ void load8_w(const void* W, bool bf16, int64_t idx, float w[8]) {
    if (bf16) {
        const uint4 v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(W) + idx);
        const uint32_t p[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            w[2 * i] = __uint_as_float(p[i] << 16);
            w[2 * i + 1] = __uint_as_float(p[i] & 0xFFFF0000u);
        }
    } else {
        const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(W) + idx);
        const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(W) + idx + 4);
        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
        w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
    }
}

// Rows of an fp32 [rows, BN] tile that fit `bytes` of LDS: the largest
// power-of-two slice of BM that is a multiple of 32 (0: none).
constexpr int rows_per_pass(int BM, int BN, int bytes) {
    int r = BM;
    while (r > 32 && r * BN * 4 > bytes) r /= 2;
    return (r * BN * 4 <= bytes && BM % r == 0 && r % 32 == 0) ? r : 0;
}

// Accumulator rows [r0, r0 + RPP) of this wavefront's sub-tile into the
// row-major fp32 LDS tile Gs [RPP, BN].  Accumulator r of 32 x 32 block
// (tm, tn) holds row 8 (r / 4) + 4 (lane / 32) + r % 4, column lane % 32; a
// 32-row block lies wholly inside or outside a pass.
template <int BN, int WM, int WN, int TM, int TN, int RPP>
__device__ __forceinline__ void stage_acc_rows(floatx16 (&acc)[TM][TN], float* Gs, int r0, int wm, int wn,
                                               int lane) {
    const int half = lane >> 5, cl = lane & 31;
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
        const int rb = wm * WM + tm * 32 - r0;
        if (rb >= 0 && rb < RPP) {
#pragma unroll
            for (int tn = 0; tn < TN; ++tn)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    Gs[(rb + (r >> 2) * 8 + half * 4 + (r & 3)) * BN + wn * WN + tn * 32 + cl] = acc[tm][tn][r];
        }
    }
}

// Inputs of one 8-weight chunk of the fused epilogue.
struct SteChunk {
    float w[8], v[8];
    float mx, mn, al, be;
    int64_t idx, gi;
    bool ok;
};

template <int BM, int BN, int NT, int WM, int WN, int TM, int TN, int LDS_BYTES>
__device__ __forceinline__ void epilogue_ste(const GemmArgs& a, const StepView& stv, floatx16 (&acc)[TM][TN],
                                             int64_t m0, int64_t n0, int wm, int wn, int lane, char* smem) {
    constexpr int RPP = rows_per_pass(BM, BN, LDS_BYTES);            // rows per pass
    static_assert(RPP > 0, "tile does not fit the fused epilogue");
    constexpr int CPR = BN / 8;                                        // chunks per row
    constexpr int NCH = RPP * CPR;                                     // chunks per pass
    static_assert(NCH % NT == 0 && 64 % CPR == 0, "chunk mapping");
    const FusedUpdate& f = a.fu;
    float* Gs = reinterpret_cast<float*>(smem);
    const int src = stv.src, dst = stv.dst, t = stv.t;
    const float lr = f.lr[t], lrc = f.lr_clip[t];
    const QParams qp = f.qp;   // a local copy: a reference into the kernel arguments spills them
    const float Q = qp.qmax;
    const int lpg = qp.group >> 3;
    const float* Vs = f.V[src];
    float* Vd = f.V[dst];

    // W, V and the group parameters of a chunk; issued one chunk ahead so
    // the HBM reads overlap the arithmetic of the previous chunk.
    auto load_chunk = [&](int r0, int c, SteChunk& in) {
        const int row = c / CPR, ch = c - row * CPR;
        const int64_t n = m0 + r0 + row, k = n0 + ch * 8;
        in.ok = n < a.I && k < a.J;
        in.idx = n * f.K + k;
        if (in.ok) {
            in.gi = n * f.G + k / f.qp.group;
            in.mx = f.mx[in.gi];
            in.mn = f.mn[in.gi];
            in.al = f.alpha[src][in.gi];
            in.be = f.beta[src][in.gi];
            load8_w(f.W, f.w_bf16, in.idx, in.w);
            const float4 v0 = *reinterpret_cast<const float4*>(Vs + in.idx);
            const float4 v1 = *reinterpret_cast<const float4*>(Vs + in.idx + 4);
            in.v[0] = v0.x; in.v[1] = v0.y; in.v[2] = v0.z; in.v[3] = v0.w;
            in.v[4] = v1.x; in.v[5] = v1.y; in.v[6] = v1.z; in.v[7] = v1.w;
        }
    };

    SteChunk cur, nxt;
    load_chunk(0, threadIdx.x, cur);
    __syncthreads();   // every wavefront is done with the operand stages
#pragma unroll 1
    for (int r0 = 0; r0 < BM; r0 += RPP) {
        stage_acc_rows<BN, WM, WN, TM, TN, RPP>(acc, Gs, r0, wm, wn, lane);
        __syncthreads();
#pragma unroll 1
        for (int c = threadIdx.x; c < NCH; c += NT) {
            // prefetch the next chunk (the first chunk of the next pass at the end)
            if (c + NT < NCH) load_chunk(r0, c + NT, nxt);
            else if (r0 + RPP < BM) load_chunk(r0 + RPP, threadIdx.x, nxt);
            const int row = c / CPR, ch = c - row * CPR;
            float sa = 0.0f, sb = 0.0f;
            float vn[8];
            if (cur.ok) {
                const GroupQ gq = group_quant(cur.mx, cur.mn, cur.al, cur.be, qp);
                float g[8];
                const float4 g0 = *reinterpret_cast<const float4*>(Gs + row * BN + ch * 8);
                const float4 g1 = *reinterpret_cast<const float4*>(Gs + row * BN + ch * 8 + 4);
                g[0] = g0.x; g[1] = g0.y; g[2] = g0.z; g[3] = g0.w;
                g[4] = g1.x; g[5] = g1.y; g[6] = g1.z; g[7] = g1.w;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    float u, ru;
                    const float ws = scaled_weight(cur.w[i], cur.v[i], gq.s, gq.r, gq.thr, u, ru);
                    const float tt = ru + gq.z;
                    const float q = __builtin_amdgcn_fmed3f(tt, 0.0f, Q);
                    const bool m = q == tt;
                    ste_terms(g[i], q, gq.z, ws, gq.wmin_s, m, sa, sb);
                    vn[i] = v_step(cur.v[i], g[i], gq.s, m, lr);
                }
            }
            for (int off = 1; off < lpg; off <<= 1) {
                sa += __shfl_xor(sa, off, 64);
                sb += __shfl_xor(sb, off, 64);
            }
            if (cur.ok) {
                float da, db;
                ste_group_grads(cur.mx, cur.mn, qp, sa, sb, da, db);
                const float an = sign_step(cur.al, da, lrc, f.clip_lo, f.clip_hi);
                const float bn = sign_step(cur.be, db, lrc, f.clip_lo, f.clip_hi);
                if ((ch & (lpg - 1)) == 0) {
                    f.alpha[dst][cur.gi] = an;
                    f.beta[dst][cur.gi] = bn;
                }
                *reinterpret_cast<float4*>(Vd + cur.idx) = make_float4(vn[0], vn[1], vn[2], vn[3]);
                *reinterpret_cast<float4*>(Vd + cur.idx + 4) = make_float4(vn[4], vn[5], vn[6], vn[7]);
                const GroupQ gn = group_quant(cur.mx, cur.mn, an, bn, qp);
                uint32_t o[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float t0, t1;
                    const float q0 = quant_code(cur.w[2 * i], vn[2 * i], gn, Q, t0);
                    const float q1 = quant_code(cur.w[2 * i + 1], vn[2 * i + 1], gn, Q, t1);
                    o[i] = pack_bf16x2(gn.s * (q0 - gn.z), gn.s * (q1 - gn.z));
                }
                *reinterpret_cast<uint4*>(f.what_next + cur.idx) = make_uint4(o[0], o[1], o[2], o[3]);
            }
            cur = nxt;
        }
        __syncthreads();
    }
}

// Fused epilogue for bf16 W with a DMA ring: the V (2 x 16 B), W (16 B) and
// group values (mx, mn, alpha, beta: 4 x 4 B) of each thread's 8-weight
// chunks are moved by global_load_lds into one of RING_SLOTS LDS slots, two
// chunks ahead of the arithmetic, so the HBM reads of three chunks per
// thread overlap without holding registers.  Lane l of a wavefront owns
// bytes [16 l, 16 l + 16) of each 1 KB part of its 4 KB slot area (V low, V
// high, W) and [4 l, 4 l + 4) of each 256 B group-value part.  Waits are
// explicit: vector-memory loads (LDS-direct ones included) complete in issue
// order, so vmcnt <= (loads issued after chunk j) means chunk j has landed,
// whatever the interleaved stores do (they only add to the count).  The
// arithmetic per chunk is that of epilogue_ste.
// Sum over aligned groups of lpg lanes (a power of two up to 64), every lane
// of a group receiving the group's sum.  The first four steps use DPP lane
// moves (xor 1 and xor 2 within quads, then the mirrored lane of the other
// quad, then of the other half-row), the rest lane shuffles.  After each
// step every lane of the partial group holds the same value, so each step
// adds exactly the operands of the xor butterfly x += x[lane ^ 2^i], and the
// result is that butterfly's bit for bit.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_group_sum(float x, int lpg) {
    if (lpg >= 2) x += dpp_move<0xB1>(x);     // quad_perm [1, 0, 3, 2]
    if (lpg >= 4) x += dpp_move<0x4E>(x);     // quad_perm [2, 3, 0, 1]
    if (lpg >= 8) x += dpp_move<0x141>(x);    // row_half_mirror
    if (lpg >= 16) x += dpp_move<0x140>(x);   // row_mirror
    if (lpg >= 32) x += __shfl_xor(x, 16, 64);
    if (lpg >= 64) x += __shfl_xor(x, 32, 64);
    return x;
}

typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

// This lane's part of a ring slot (slot base b is wave-uniform): three
// 16-byte and four 4-byte LDS reads, waited for in the same statement.  The
// caller has waited (vmcnt) for the DMA that filled the slot; reading through
// one asm statement keeps the compiler from adding its own, coarser wait.
__device__ __forceinline__ void ring_read(const char* b, int lane, const float* gp, f32x4v& v0, f32x4v& v1,
                                          u32x4v& w, float& mx, float& mn, float& al, float& be, f32x4v& g0,
                                          f32x4v& g1) {
    const uint32_t a16 = (uint32_t)(uintptr_t)(lds_void*)(b + lane * 16);
    const uint32_t a4 = (uint32_t)(uintptr_t)(lds_void*)(b + lane * 4);
    const uint32_t ag = (uint32_t)(uintptr_t)(lds_void*)gp;
    asm volatile(
        "ds_read_b128 %0, %9\n\t"
        "ds_read_b128 %1, %9 offset:1024\n\t"
        "ds_read_b128 %2, %9 offset:2048\n\t"
        "ds_read_b32 %3, %10 offset:3072\n\t"
        "ds_read_b32 %4, %10 offset:3328\n\t"
        "ds_read_b32 %5, %10 offset:3584\n\t"
        "ds_read_b32 %6, %10 offset:3840\n\t"
        "ds_read_b128 %7, %11\n\t"
        "ds_read_b128 %8, %11 offset:16\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v0), "=&v"(v1), "=&v"(w), "=&v"(mx), "=&v"(mn), "=&v"(al), "=&v"(be), "=&v"(g0), "=&v"(g1)
        : "v"(a16), "v"(a4), "v"(ag)
        : "memory");
}

// Accumulator rows [r0, r0 + RPP) into the G tile like stage_acc_rows, as
// ds_write_b32 statements the compiler does not track (see ring_read).
template <int BN, int WM, int WN, int TM, int TN, int RPP>
__device__ __forceinline__ void stage_acc_rows_asm(floatx16 (&acc)[TM][TN], const char* gsm, int r0, int wm,
                                                   int wn, int lane) {
    const int half = lane >> 5, cl = lane & 31;
    const uint32_t lbase = (uint32_t)(uintptr_t)(lds_void*)gsm + (uint32_t)(((half * 4) * BN + wn * WN + cl) * 4);
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
        const int rb = wm * WM + tm * 32 - r0;
        if (rb >= 0 && rb < RPP) {
            const uint32_t ab = lbase + (uint32_t)(rb * BN * 4);
#pragma unroll
            for (int tn = 0; tn < TN; ++tn)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    asm volatile("ds_write_b32 %0, %1 offset:%2"
                                 :
                                 : "v"(ab), "v"(acc[tm][tn][r]), "n"((((r >> 2) * 8 + (r & 3)) * BN + tn * 32) * 4)
                                 : "memory");
                }
        }
    }
}

constexpr int RING_SLOTS = 3;
constexpr int RING_WAVE_BYTES = 4096;
constexpr int RING_LOADS = 7;                   // loads per chunk
// GL > 0: asymmetric groups of 8 GL weights, known at compile time, so the
// group sums are straight-line lane moves and no branch tests the mapping;
// GL = 0 reads both from the quantizer parameters.
// CHUNK_TIES: the near-tie tests of a chunk's eight weights share one branch
// into the division path instead of one branch per weight.
template <int BM, int BN, int NT, int WM, int WN, int TM, int TN, int GBYTES, int GL = 0, bool CHUNK_TIES = false>
__device__ __forceinline__ void epilogue_ste_ring(const GemmArgs& a, const StepView& stv, floatx16 (&acc)[TM][TN],
                                                  int64_t m0, int64_t n0, int wm, int wn, int lane, char* gsm,
                                                  char* q0, char* q1, char* q2) {
    constexpr int RPP = rows_per_pass(BM, BN, GBYTES);
    static_assert(RPP > 0, "tile does not fit the fused epilogue");
    constexpr int CPR = BN / 8;                 // chunks per row
    constexpr int NCH = RPP * CPR;              // chunks per pass
    static_assert(NCH % NT == 0 && 64 % CPR == 0, "chunk mapping");
    constexpr int CPT = NCH / NT;               // chunks per thread per pass
    constexpr int NJ = (BM / RPP) * CPT;        // chunks per thread
    constexpr int AHEAD = RING_SLOTS - 1;
    const FusedUpdate& f = a.fu;
    float* Gs = reinterpret_cast<float*>(gsm);
    // the step's scalars, in scalar registers before any ring load is issued
    const int src = __builtin_amdgcn_readfirstlane(stv.src);
    const int dst = __builtin_amdgcn_readfirstlane(stv.dst);
    const int t = __builtin_amdgcn_readfirstlane(stv.t);
    const float lr = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, f.lr[t])));
    const float lrc =
        __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, f.lr_clip[t])));
    QParams qp = f.qp;   // a local copy: a reference into the kernel arguments spills them
    if constexpr (GL > 0) qp.sym = 0;
    constexpr bool BATCH_TIES = CHUNK_TIES;
    const float Q = qp.qmax;
    const int lpg = GL > 0 ? GL : (qp.group >> 3);
    const float* Vs = f.V[src];
    float* Vd = f.V[dst];
    const uint16_t* Wb = static_cast<const uint16_t*>(f.W);
    const float* Als = f.alpha[src];
    const float* Bes = f.beta[src];
    const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int tix = wv * 64 + lane;
    const int woff = wv * RING_WAVE_BYTES;
    auto slot = [&](auto J) -> char* {
        constexpr int i = decltype(J)::value % RING_SLOTS;
        if constexpr (i == 0) return q0 + woff;
        else if constexpr (i == 1) return q1 + woff;
        else return q2 + woff;
    };
    // Position of chunk j of this thread (j a compile-time constant): the
    // column chunk is the same for all of a thread's chunks (NT is a
    // multiple of CPR), the row advances by a compile-time step.
    static_assert(NT % CPR == 0, "chunk columns per thread");
    const int ch0 = tix % CPR, row0 = tix / CPR;
    const int64_t k0 = n0 + ch0 * 8;
    const bool kok = k0 < a.J;
    const int64_t n00 = m0 + row0;
    const int64_t idx00 = n00 * f.K + k0, gi00 = n00 * f.G + k0 / f.qp.group;
    struct Pos {
        int64_t idx, gi;
        int ch;
        bool ok;
    };
    auto pos = [&](auto J) -> Pos {
        constexpr int j = decltype(J)::value;
        constexpr int pass = j / CPT, within = j % CPT;
        constexpr int drow = pass * RPP + within * (NT / CPR);
        Pos q;
        q.ch = ch0;
        q.ok = kok && n00 + drow < a.I;
        q.idx = q.ok ? idx00 + (int64_t)drow * f.K : 0;
        q.gi = q.ok ? gi00 + (int64_t)drow * f.G : 0;
        return q;
    };
    // RING_LOADS unconditional loads per chunk (out-of-range lanes read element 0)
    auto issue = [&](auto J) {
        const Pos q = pos(J);
        char* b = slot(J);
        __builtin_amdgcn_global_load_lds((gbl_void*)(Vs + q.idx), (lds_void*)b, 16, 0, 0);
        __builtin_amdgcn_global_load_lds((gbl_void*)(Vs + q.idx + 4), (lds_void*)(b + 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((gbl_void*)(Wb + q.idx), (lds_void*)(b + 2048), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((gbl_void*)(f.mx + q.gi), (lds_void*)(b + 3072), 4, 0, 0);
        __builtin_amdgcn_global_load_lds((gbl_void*)(f.mn + q.gi), (lds_void*)(b + 3328), 4, 0, 0);
        __builtin_amdgcn_global_load_lds((gbl_void*)(Als + q.gi), (lds_void*)(b + 3584), 4, 0, 0);
        __builtin_amdgcn_global_load_lds((gbl_void*)(Bes + q.gi), (lds_void*)(b + 3840), 4, 0, 0);
    };
    auto process = [&](auto J) {
        constexpr int j = decltype(J)::value;
        constexpr int pass = j / CPT, within = j % CPT;
        if constexpr (within == 0) {
            lds_barrier();                       // the previous pass's G tile is read
            stage_acc_rows_asm<BN, WM, WN, TM, TN, RPP>(acc, gsm, pass * RPP, wm, wn, lane);
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        }
        // chunk j landed: at most the loads of the chunks issued after it remain
        constexpr int later = (NJ - 1 - j) < AHEAD ? (NJ - 1 - j) : AHEAD;
        wait_vmcnt<RING_LOADS * later>();
        const Pos q = pos(J);
        const int row = row0 + within * (NT / CPR), ch = q.ch;
        f32x4v v0, v1, g0, g1;
        u32x4v wr;
        float pmx, pmn, pal, pbe;
        ring_read(slot(J), lane, Gs + row * BN + ch * 8, v0, v1, wr, pmx, pmn, pal, pbe, g0, g1);
        const float vv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
        const uint32_t wu[4] = {wr.x, wr.y, wr.z, wr.w};
        float w[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            w[2 * i] = bf16_to_f32((uint16_t)(wu[i] & 0xffffu));
            w[2 * i + 1] = bf16_to_f32((uint16_t)(wu[i] >> 16));
        }
        float sa = 0.0f, sb = 0.0f;
        float vn[8];
        if (q.ok) {
            const GroupQ gq = group_quant(pmx, pmn, pal, pbe, qp);
            const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
            auto terms = [&](int i, float ws, float ru) {
                const float tt = ru + gq.z;
                const float qq = __builtin_amdgcn_fmed3f(tt, 0.0f, Q);
                const bool m = qq == tt;
                ste_terms(g[i], qq, gq.z, ws, gq.wmin_s, m, sa, sb);
                vn[i] = v_step(vv[i], g[i], gq.s, m, lr);
            };
            if constexpr (BATCH_TIES) {
                float wsv[8], ruv[8];
                scaled_weights8(w, vv, gq.s, gq.r, gq.thr, wsv, ruv);
#pragma unroll
                for (int i = 0; i < 8; ++i) terms(i, wsv[i], ruv[i]);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    float u, ru;
                    const float ws = scaled_weight(w[i], vv[i], gq.s, gq.r, gq.thr, u, ru);
                    terms(i, ws, ru);
                }
            }
        }
        sa = lane_group_sum(sa, lpg);
        sb = lane_group_sum(sb, lpg);
        if (q.ok) {
            float da, db;
            ste_group_grads(pmx, pmn, qp, sa, sb, da, db);
            const float an = sign_step(pal, da, lrc, f.clip_lo, f.clip_hi);
            const float bn = sign_step(pbe, db, lrc, f.clip_lo, f.clip_hi);
            if ((ch & (lpg - 1)) == 0) {
                f.alpha[dst][q.gi] = an;
                f.beta[dst][q.gi] = bn;
            }
            // the updated V and the next w^ are read again only in the next
            // step: non-temporal stores keep them from displacing this
            // epilogue's loads in the caches (70B block 7.94 -> 7.80 ms)
            __builtin_nontemporal_store(f32x4v{vn[0], vn[1], vn[2], vn[3]}, reinterpret_cast<f32x4v*>(Vd + q.idx));
            __builtin_nontemporal_store(f32x4v{vn[4], vn[5], vn[6], vn[7]}, reinterpret_cast<f32x4v*>(Vd + q.idx + 4));
            const GroupQ gn = group_quant(pmx, pmn, an, bn, qp);
            uint32_t o[4];
            if constexpr (BATCH_TIES) {
                float wsn[8], run[8];
                scaled_weights8(w, vn, gn.s, gn.r, gn.thr, wsn, run);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float c0 = __builtin_amdgcn_fmed3f(run[2 * i] + gn.z, 0.0f, Q);
                    const float c1 = __builtin_amdgcn_fmed3f(run[2 * i + 1] + gn.z, 0.0f, Q);
                    o[i] = pack_bf16x2(gn.s * (c0 - gn.z), gn.s * (c1 - gn.z));
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float t0, t1;
                    const float c0 = quant_code(w[2 * i], vn[2 * i], gn, Q, t0);
                    const float c1 = quant_code(w[2 * i + 1], vn[2 * i + 1], gn, Q, t1);
                    o[i] = pack_bf16x2(gn.s * (c0 - gn.z), gn.s * (c1 - gn.z));
                }
            }
            __builtin_nontemporal_store(u32x4v{o[0], o[1], o[2], o[3]}, reinterpret_cast<u32x4v*>(f.what_next + q.idx));
        }
    };
    lds_barrier();   // every wavefront is done with the operand stages
    static_for<(NJ < AHEAD ? NJ : AHEAD)>([&](auto J) { issue(J); });
    static_for<NJ>([&](auto J) {
        constexpr int j = decltype(J)::value;
        if constexpr (j + AHEAD < NJ) issue(std::integral_constant<int, j + AHEAD>{});
        process(J);
    });
}

// LDS-staged epilogue of the LDS-direct kernels (EPI_STORE and EPI_LOSS):
// the accumulators go to the idle operand LDS, RPP rows at a time, and are
// read back row-major so each thread owns 8 consecutive columns: the
// reference values are read and C / dY^T written as 16-32 byte vectors along
// contiguous columns (needs J % 8 == 0; columns of one sample are contiguous
// in the reference because T % 8 == 0).
template <int BM, int BN, int NT, int WM, int WN, int TM, int TN, int EPI, int LDS_BYTES>
__device__ __forceinline__ void epilogue_lds(const GemmArgs& a, const SchedView& sv, floatx16 (&acc)[TM][TN],
                                             int64_t m0, int64_t n0, int wm, int wn, int lane, char* smem,
                                             double* red, float* out) {
    constexpr int RPP = rows_per_pass(BM, BN, LDS_BYTES);
    static_assert(RPP > 0, "tile does not fit the LDS epilogue");
    constexpr int CPR = BN / 8;
    static_assert((RPP * CPR) % NT == 0 && 64 % CPR == 0, "chunk mapping");
    constexpr int NPASS = BM / RPP, CPT = RPP * CPR / NT;   // passes; chunks per thread and pass
    // The loss epilogue loads every reference-output chunk of the tile before
    // the first pass, so their HBM latency overlaps the staging of the
    // accumulators instead of following each pass's barrier.
    constexpr bool PRE = EPI == EPI_LOSS && NPASS * CPT <= 8;
    float* Cs = reinterpret_cast<float*>(smem);
    float lsum = 0.0f;
    float4 ypre[PRE ? NPASS : 1][PRE ? CPT : 1][2];
    auto yref_ptr = [&](int64_t i, int64_t j) {
        const int64_t seg = j / a.yref_T;
        return a.yref + sv.id(seg) * a.yref_seg_stride + i * a.yref_ld + (j - seg * a.yref_T);
    };
    if constexpr (PRE) {
#pragma unroll
        for (int p = 0; p < NPASS; ++p)
#pragma unroll
            for (int q = 0; q < CPT; ++q) {
                const int c = (int)threadIdx.x + q * NT;
                const int row = c / CPR, ch = c - row * CPR;
                const int64_t i = m0 + p * RPP + row, j = n0 + ch * 8;
                if (i < a.I && j < a.J) {
                    const float* y = yref_ptr(i, j);
                    ypre[p][q][0] = *reinterpret_cast<const float4*>(y);
                    ypre[p][q][1] = *reinterpret_cast<const float4*>(y + 4);
                }
            }
    }
    __syncthreads();   // every wavefront is done with the operand stages
    auto pass = [&](int p) {
        const int r0 = p * RPP;
        stage_acc_rows<BN, WM, WN, TM, TN, RPP>(acc, Cs, r0, wm, wn, lane);
        __syncthreads();
#pragma unroll
        for (int q = 0; q < CPT; ++q) {
            const int c = (int)threadIdx.x + q * NT;
            const int row = c / CPR, ch = c - row * CPR;
            const int64_t i = m0 + r0 + row, j = n0 + ch * 8;
            if (i >= a.I || j >= a.J) continue;
            const float4 c0 = *reinterpret_cast<const float4*>(Cs + row * BN + ch * 8);
            const float4 c1 = *reinterpret_cast<const float4*>(Cs + row * BN + ch * 8 + 4);
            if (EPI == EPI_STORE) {
                float* o = out + i * a.ldc + j;
                *reinterpret_cast<float4*>(o) = c0;
                *reinterpret_cast<float4*>(o + 4) = c1;
            } else {
                float4 y0, y1;
                if constexpr (PRE) {
                    y0 = ypre[PRE ? p : 0][PRE ? q : 0][0];
                    y1 = ypre[PRE ? p : 0][PRE ? q : 0][1];
                } else {
                    const float* y = yref_ptr(i, j);
                    y0 = *reinterpret_cast<const float4*>(y);
                    y1 = *reinterpret_cast<const float4*>(y + 4);
                }
                const float d[8] = {c0.x - y0.x, c0.y - y0.y, c0.z - y0.z, c0.w - y0.w,
                                    c1.x - y1.x, c1.y - y1.y, c1.z - y1.z, c1.w - y1.w};
#pragma unroll
                for (int e = 0; e < 8; ++e) lsum += d[e] * d[e];
                if (a.dyt_bf16) {
                    uint32_t o[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        o[e] = (uint32_t)f32_to_bf16(a.dscale * d[2 * e]) |
                               ((uint32_t)f32_to_bf16(a.dscale * d[2 * e + 1]) << 16);
                    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.dyt) + i * a.lddyt + j) =
                        make_uint4(o[0], o[1], o[2], o[3]);
                } else {
                    float* o = static_cast<float*>(a.dyt) + i * a.lddyt + j;
                    *reinterpret_cast<float4*>(o) = make_float4(a.dscale * d[0], a.dscale * d[1], a.dscale * d[2],
                                                                a.dscale * d[3]);
                    *reinterpret_cast<float4*>(o + 4) = make_float4(a.dscale * d[4], a.dscale * d[5],
                                                                    a.dscale * d[6], a.dscale * d[7]);
                }
            }
        }
        __syncthreads();
    };
    if constexpr (PRE) {
#pragma unroll
        for (int p = 0; p < NPASS; ++p) pass(p);
    } else {
#pragma unroll 1
        for (int p = 0; p < NPASS; ++p) pass(p);
    }
    if (EPI == EPI_LOSS) {
        double v = (double)lsum;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
        if (lane == 0) red[threadIdx.x >> 6] = v;
    }
}

// ------------------------------------------------------------------ bf16 --
template <int BM, int BN, int BK, int NWM, int NWN, int EPI>
__global__ void __launch_bounds__(NWM * NWN * 64) gemm_bf16_kernel(GemmArgs a) {
    constexpr int NW = NWM * NWN;
    constexpr int NT = NW * 64;
    constexpr int WM = BM / NWM, WN = BN / NWN;
    constexpr int TM = WM / 32, TN = WN / 32;
    constexpr int PITCH = BK + 8;            // bf16 elements per LDS row
    constexpr int CPR = BK / 8;              // 16-byte chunks per row
    constexpr int AC = BM * CPR / NT, BC = BN * CPR / NT;
    constexpr int KS = BK / 16;              // MFMA sub-steps per BK step
    static_assert(AC * NT == BM * CPR && BC * NT == BN * CPR, "tile/thread mismatch");
    static_assert(TM >= 1 && TN >= 1, "wavefront tile below one MFMA block");
    __shared__ __attribute__((aligned(16))) uint16_t smem[2][(BM + BN) * PITCH];
    __shared__ double red[NW];

    if (a.state && a.state->halted) return;
    const StepView stv = step_view(a);
    const SchedView sv = sched_view(a, stv.row);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / NWN, wn = wave % NWN;
    const int64_t tiles_m = (a.I + BM - 1) / BM, tiles_n = (a.J + BN - 1) / BN;
    int64_t tile_m, tile_n;
    tile_coords<BM, BN>(tiles_m, tiles_n, tile_m, tile_n);
    const int64_t m0 = tile_m * BM, n0 = tile_n * BN;
    const bool full = (m0 + BM <= a.I) && (n0 + BN <= a.J) && (a.R % BK == 0);

    const uint16_t* Ab = static_cast<const uint16_t*>(a.A.base);
    const uint16_t* Bb = static_cast<const uint16_t*>(a.B.base);
    int64_t aoff[AC], boff[BC];
#pragma unroll
    for (int q = 0; q < AC; ++q) {
        const int c = tid + q * NT;
        const int64_t i = m0 + c / CPR;
        aoff[q] = (i < a.I) ? row_offset(a.A, sv, i) + (c % CPR) * 8 : -1;
    }
#pragma unroll
    for (int q = 0; q < BC; ++q) {
        const int c = tid + q * NT;
        const int64_t j = n0 + c / CPR;
        boff[q] = (j < a.J) ? row_offset(a.B, sv, j) + (c % CPR) * 8 : -1;
    }

    uint4 ra[AC], rb[BC];
    auto gload = [&](int64_t k0) {
        const int64_t ca = col_offset(a.A, sv, k0), cb = col_offset(a.B, sv, k0);
        if (full) {
#pragma unroll
            for (int q = 0; q < AC; ++q) ra[q] = *reinterpret_cast<const uint4*>(Ab + aoff[q] + ca);
#pragma unroll
            for (int q = 0; q < BC; ++q) rb[q] = *reinterpret_cast<const uint4*>(Bb + boff[q] + cb);
        } else {
#pragma unroll
            for (int q = 0; q < AC; ++q) {
                const int kk = ((tid + q * NT) % CPR) * 8;
                ra[q] = (aoff[q] >= 0 && k0 + kk < a.R) ? *reinterpret_cast<const uint4*>(Ab + aoff[q] + ca)
                                                         : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int q = 0; q < BC; ++q) {
                const int kk = ((tid + q * NT) % CPR) * 8;
                rb[q] = (boff[q] >= 0 && k0 + kk < a.R) ? *reinterpret_cast<const uint4*>(Bb + boff[q] + cb)
                                                         : make_uint4(0, 0, 0, 0);
            }
        }
    };
    auto sstore = [&](int buf) {
        uint16_t* As = smem[buf];
        uint16_t* Bs = smem[buf] + BM * PITCH;
#pragma unroll
        for (int q = 0; q < AC; ++q) {
            const int c = tid + q * NT;
            *reinterpret_cast<uint4*>(As + (c / CPR) * PITCH + (c % CPR) * 8) = ra[q];
        }
#pragma unroll
        for (int q = 0; q < BC; ++q) {
            const int c = tid + q * NT;
            *reinterpret_cast<uint4*>(Bs + (c / CPR) * PITCH + (c % CPR) * 8) = rb[q];
        }
    };

    floatx16 acc[TM][TN];
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[tm][tn][r] = 0.0f;

    const int64_t nk = (a.R + BK - 1) / BK;
    gload(0);
    sstore(0);
    __syncthreads();
    const int frow = lane & 31, fk = (lane >> 5) * 8;
    for (int64_t kt = 0; kt < nk; ++kt) {
        const int buf = (int)(kt & 1);
        if (kt + 1 < nk) gload((kt + 1) * BK);
        const uint16_t* As = smem[buf] + (wm * WM + frow) * PITCH + fk;
        const uint16_t* Bs = smem[buf] + BM * PITCH + (wn * WN + frow) * PITCH + fk;
        bf16x8 af[2][TM], bfr[2][TN];
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) af[0][tm] = *reinterpret_cast<const bf16x8*>(As + tm * 32 * PITCH);
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) bfr[0][tn] = *reinterpret_cast<const bf16x8*>(Bs + tn * 32 * PITCH);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int cb = ks & 1, nb = cb ^ 1;
            if (ks + 1 < KS) {
#pragma unroll
                for (int tm = 0; tm < TM; ++tm)
                    af[nb][tm] = *reinterpret_cast<const bf16x8*>(As + tm * 32 * PITCH + (ks + 1) * 16);
#pragma unroll
                for (int tn = 0; tn < TN; ++tn)
                    bfr[nb][tn] = *reinterpret_cast<const bf16x8*>(Bs + tn * 32 * PITCH + (ks + 1) * 16);
            }
#pragma unroll
            for (int tm = 0; tm < TM; ++tm)
#pragma unroll
                for (int tn = 0; tn < TN; ++tn)
                    acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cb][tm], bfr[cb][tn], acc[tm][tn], 0, 0, 0);
        }
        if (kt + 1 < nk) sstore(buf ^ 1);
        __syncthreads();
    }

    epilogue<TM, TN, EPI>(a, sv, acc, m0 + wm * WM, n0 + wn * WN, lane, red);
    if (EPI == EPI_LOSS) {
        __syncthreads();
        if (tid == 0) {
            double s = 0.0;
            for (int w = 0; w < NW; ++w) s += red[w];
            a.partials[blockIdx.x] = s;
        }
    }
}

// ------------------------------------------------------------------ fp32 --
template <int BM, int BN, int BK, int NWM, int NWN, int EPI>
__global__ void __launch_bounds__(NWM * NWN * 64) gemm_f32_kernel(GemmArgs a) {
    constexpr int NW = NWM * NWN;
    constexpr int NT = NW * 64;
    constexpr int WM = BM / NWM, WN = BN / NWN;
    constexpr int TM = WM / 32, TN = WN / 32;
    constexpr int PITCH = BK + 4;            // floats per LDS row
    constexpr int CPR = BK / 4;              // 16-byte chunks per row
    constexpr int AC = BM * CPR / NT, BC = BN * CPR / NT;
    static_assert(AC * NT == BM * CPR && BC * NT == BN * CPR, "tile/thread mismatch");
    __shared__ __attribute__((aligned(16))) float smem[2][(BM + BN) * PITCH];
    __shared__ double red[NW];

    if (a.state && a.state->halted) return;
    const StepView stv = step_view(a);
    const SchedView sv = sched_view(a, stv.row);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / NWN, wn = wave % NWN;
    const int64_t tiles_m = (a.I + BM - 1) / BM, tiles_n = (a.J + BN - 1) / BN;
    int64_t tile_m, tile_n;
    tile_coords<BM, BN>(tiles_m, tiles_n, tile_m, tile_n);
    const int64_t m0 = tile_m * BM, n0 = tile_n * BN;

    const float* Ab = static_cast<const float*>(a.A.base);
    const float* Bb = static_cast<const float*>(a.B.base);
    int64_t aoff[AC], boff[BC];
#pragma unroll
    for (int q = 0; q < AC; ++q) {
        const int c = tid + q * NT;
        const int64_t i = m0 + c / CPR;
        aoff[q] = (i < a.I) ? row_offset(a.A, sv, i) + (c % CPR) * 4 : -1;
    }
#pragma unroll
    for (int q = 0; q < BC; ++q) {
        const int c = tid + q * NT;
        const int64_t j = n0 + c / CPR;
        boff[q] = (j < a.J) ? row_offset(a.B, sv, j) + (c % CPR) * 4 : -1;
    }
    float4 ra[AC], rb[BC];
    auto gload = [&](int64_t k0) {
        const int64_t ca = col_offset(a.A, sv, k0), cb = col_offset(a.B, sv, k0);
#pragma unroll
        for (int q = 0; q < AC; ++q) {
            const int kk = ((tid + q * NT) % CPR) * 4;
            ra[q] = (aoff[q] >= 0 && k0 + kk < a.R) ? *reinterpret_cast<const float4*>(Ab + aoff[q] + ca)
                                                     : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int q = 0; q < BC; ++q) {
            const int kk = ((tid + q * NT) % CPR) * 4;
            rb[q] = (boff[q] >= 0 && k0 + kk < a.R) ? *reinterpret_cast<const float4*>(Bb + boff[q] + cb)
                                                     : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };
    auto sstore = [&](int buf) {
        float* As = smem[buf];
        float* Bs = smem[buf] + BM * PITCH;
#pragma unroll
        for (int q = 0; q < AC; ++q) {
            const int c = tid + q * NT;
            *reinterpret_cast<float4*>(As + (c / CPR) * PITCH + (c % CPR) * 4) = ra[q];
        }
#pragma unroll
        for (int q = 0; q < BC; ++q) {
            const int c = tid + q * NT;
            *reinterpret_cast<float4*>(Bs + (c / CPR) * PITCH + (c % CPR) * 4) = rb[q];
        }
    };

    floatx16 acc[TM][TN];
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[tm][tn][r] = 0.0f;

    const int64_t nk = (a.R + BK - 1) / BK;
    gload(0);
    sstore(0);
    __syncthreads();
    const int frow = lane & 31, fk = lane >> 5;
    for (int64_t kt = 0; kt < nk; ++kt) {
        const int buf = (int)(kt & 1);
        if (kt + 1 < nk) gload((kt + 1) * BK);
        const float* As = smem[buf] + (wm * WM + frow) * PITCH + fk;
        const float* Bs = smem[buf] + BM * PITCH + (wn * WN + frow) * PITCH + fk;
#pragma unroll
        for (int ks = 0; ks < BK; ks += 2) {
            float af[TM], bfr[TN];
#pragma unroll
            for (int tm = 0; tm < TM; ++tm) af[tm] = As[tm * 32 * PITCH + ks];
#pragma unroll
            for (int tn = 0; tn < TN; ++tn) bfr[tn] = Bs[tn * 32 * PITCH + ks];
#pragma unroll
            for (int tm = 0; tm < TM; ++tm)
#pragma unroll
                for (int tn = 0; tn < TN; ++tn)
                    acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[tm], bfr[tn], acc[tm][tn], 0, 0, 0);
        }
        if (kt + 1 < nk) sstore(buf ^ 1);
        __syncthreads();
    }

    epilogue<TM, TN, EPI>(a, sv, acc, m0 + wm * WM, n0 + wn * WN, lane, red);
    if (EPI == EPI_LOSS) {
        __syncthreads();
        if (tid == 0) {
            double s = 0.0;
            for (int w = 0; w < NW; ++w) s += red[w];
            a.partials[blockIdx.x] = s;
        }
    }
}

// --------------------------------------------------- bf16, LDS direct ----
// Multi-stage variant: each wavefront moves 64 x 16 bytes per instruction
// straight from global memory into LDS (gfx950 global_load_lds_dwordx4), so
// STAGES-1 BK steps are in flight without holding registers.  Rows are 128
// bytes (BK = 64 bf16) and unpadded.  A 16-byte fragment read is served 16
// lanes (16 consecutive rows, one chunk) at a time across 64 four-byte
// banks, i.e. a 256-byte window holding two rows; chunk c of row r is stored
// in slot c ^ ((r / 2) % 8), so the 8 even and the 8 odd rows of such a
// group each use all 8 slots and the group hits 16 distinct bank quads.  The
// DMA writes are linear per wavefront and conflict-free.  Rows past the end of the operand
// are clamped to the last row (their results fall outside C and are never
// stored); the reduction length must be a multiple of BK.


// Wait until at most LPW * ahead of this wave's loads are outstanding
// (ahead = stages still allowed in flight, 0..MAXA; vmcnt is an immediate).
template <int LPW, int MAXA>
__device__ __forceinline__ void wait_vmcnt_upto(int ahead) {
    if constexpr (MAXA <= 0) {
        wait_vmcnt<0>();
    } else {
        if (ahead >= MAXA) wait_vmcnt<LPW * MAXA>();
        else wait_vmcnt_upto<LPW, MAXA - 1>(ahead);
    }
}

template <int BM, int BN, int BK, int NWM, int NWN, int STAGES, int EPI, int KPRE = BK / 16, bool WB16 = false,
          bool SPLIT = false, bool AT = false, bool BT = false, int GL = 0, bool CHUNK_TIES = false>
__global__ void __launch_bounds__(NWM * NWN * 64) gemm_bf16_dma_kernel(GemmArgs a) {
    static_assert(BK == 32 || BK == 64, "BK");
    static_assert(KPRE >= 1 && KPRE <= BK / 16, "fragment prefetch depth");
    constexpr int NW = NWM * NWN;
    constexpr int NT = NW * 64;
    constexpr int WM = BM / NWM, WN = BN / NWN;
    constexpr int TM = WM / 32, TN = WN / 32;
    constexpr int ROWB = BK * 2;                       // bytes per LDS row
    constexpr int SLOTS = BK / 8;                      // 16-byte chunks per row
    constexpr int RPW = 256 / ROWB;                    // rows per 256-byte bank window
    constexpr int RPL = 64 / SLOTS;                    // rows per wave-load (64 lanes x 16 B)
    constexpr int LPW = (BM + BN) / (RPL * NW);        // wave-loads per wave per stage
    static_assert(LPW * RPL * NW == BM + BN, "rows must split evenly over wavefronts");
    static_assert(BM % RPL == 0 && BN % RPL == 0, "row blocks");
    static_assert(STAGES >= 2 && STAGES <= 8, "stages");
    static_assert(LPW * (STAGES - 2) < 64, "vmcnt budget");
    // One LDS object per stage and operand: with the stage index a
    // compile-time constant in the unrolled loop below, the compiler can tell
    // the stage being read from the stages the DMA is filling and does not
    // wait for those loads.  The fused epilogue reuses them (plus sq3) as the
    // G tile and its DMA ring.
    constexpr int ABYTES = BM * ROWB, BBYTES = BN * ROWB;
    constexpr int QA = BM / (RPL * NW);                // wave-loads per wave that fill A
    static_assert(QA * RPL * NW == BM, "A rows must split evenly over wavefronts");
    // A transposed operand (AT / BT) fills the same stage bytes as BK rows of
    // the reduction, each holding the tile's BM (BN) output indices: LPR
    // lanes of a 1 KB wave-load per row, 16-byte chunk c of row r stored in
    // slot c ^ 4 (r % 4).  Its fragments are read with ds_read_b64_tr_b16.
    constexpr int ROWTA = BM * 2, ROWTB = BN * 2;     // bytes per reduction row
    constexpr int LPRA = ROWTA / 16, LPRB = ROWTB / 16;
    static_assert(BK == 64 || (!AT && !BT), "transposed operands use BK = 64");
    static_assert(!AT || (LPRA >= 16 && 64 % LPRA == 0), "transposed A tile width");
    static_assert(!BT || (LPRB >= 16 && 64 % LPRB == 0), "transposed B tile width");
    static_assert(EPI == EPI_STORE || (!AT && !BT), "transposed operands in plain-store GEMMs only");
    // (WB16: fused epilogue on bf16 weights, which the DMA ring moves)
    constexpr bool RING =
        EPI == EPI_STE && WB16 && STAGES == 2 && BBYTES >= NW * RING_WAVE_BYTES && ABYTES >= NW * RING_WAVE_BYTES;
    __shared__ __attribute__((aligned(1024))) char sa0[ABYTES];
    __shared__ __attribute__((aligned(1024))) char sb0[BBYTES];
    __shared__ __attribute__((aligned(1024))) char sa1[ABYTES];
    __shared__ __attribute__((aligned(1024))) char sb1[BBYTES];
    __shared__ __attribute__((aligned(1024))) char sa2[STAGES > 2 ? ABYTES : 16];
    __shared__ __attribute__((aligned(1024))) char sb2[STAGES > 2 ? BBYTES : 16];
    __shared__ __attribute__((aligned(1024))) char sa3[STAGES > 3 ? ABYTES : 16];
    __shared__ __attribute__((aligned(1024))) char sb3[STAGES > 3 ? BBYTES : 16];
    __shared__ double red[EPI == EPI_LOSS ? NW : 1];
    struct StageMem {
        char* A;
        char* B;
    };
    auto stage_mem = [&](auto I) -> StageMem {
        constexpr int i = decltype(I)::value;
        if constexpr (i == 0) return {sa0, sb0};
        else if constexpr (i == 1) return {sa1, sb1};
        else if constexpr (i == 2) return {sa2, sb2};
        else return {sa3, sb3};
    };
    static_assert(STAGES <= 4, "stages");

    if (a.state && a.state->halted) return;
    StepView stv = step_view(a);
    FoldPre<RING ? 4 : 0> fold_pre;
    const bool folded = EPI == EPI_STE && a.dec_partials != nullptr;
    if (folded && !fold_begin(a, stv, fold_pre)) return;
    const SchedView sv = sched_view(a, stv.row);
    // wave index in a scalar register and the lane from the exec mask, so no
    // vector register has to carry the thread id across the main loop
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lane = (int)__lane_id();
    const int tid = wave * 64 + lane;
    const int wm = wave / NWN, wn = wave % NWN;
    const int64_t tiles_m = (a.I + BM - 1) / BM, tiles_n = (a.J + BN - 1) / BN;
    int64_t tile_m, tile_n;
    tile_coords<BM, BN>(tiles_m, tiles_n, tile_m, tile_n);
    const int64_t m0 = tile_m * BM, n0 = tile_n * BN;

    // Per-lane source offsets (elements) of this wave's loads, without the
    // reduction offset.  Wave-load p covers tile rows [RPL p, RPL (p+1)) of A
    // then B; lane l fills slot l % SLOTS of row l / SLOTS.
    // SPLIT (plain store, launch_gemm_bf16_split2): blockIdx.y = 1 takes the
    // second half of the reduction, both operands starting R/2 columns in,
    // and stores its tile to out2
    static_assert(!SPLIT || EPI == EPI_STORE, "split launches store plainly");
    const int64_t Rk = SPLIT ? a.R / 2 : a.R;
    const int64_t kofs = (SPLIT && blockIdx.y == 1) ? Rk : 0;
    float* const out = (SPLIT && blockIdx.y == 1) ? a.out2 : a.out;
    const uint16_t* Ab = static_cast<const uint16_t*>(a.A.base) + (AT ? kofs * a.A.ld : kofs);
    const uint16_t* Bb = static_cast<const uint16_t*>(a.B.base) + (BT ? kofs * a.B.ld : kofs);
    int64_t goff[LPW];
#pragma unroll
    for (int q = 0; q < LPW; ++q) {
        const int p = wave + q * NW;
        const int trow = p * RPL + lane / SLOTS;       // row within the combined tile
        const int chunk = (lane % SLOTS) ^ ((trow / RPW) % SLOTS);
        if (p * RPL < BM) {
            if constexpr (AT) {
                // reduction row rr of the stage; output columns clamped to the last chunk
                const int rr = (p * 1024) / ROWTA + lane / LPRA;
                int64_t x = m0 + ((lane % LPRA) ^ (4 * (rr & 3))) * 8;
                if (x > a.I - 8) x = a.I - 8;
                goff[q] = rr * a.A.ld + x;
            } else {
                int64_t i = m0 + trow;
                if (i >= a.I) i = a.I - 1;
                goff[q] = row_offset(a.A, sv, i) + chunk * 8;
            }
        } else {
            if constexpr (BT) {
                const int rr = ((p - BM / RPL) * 1024) / ROWTB + lane / LPRB;
                int64_t x = n0 + ((lane % LPRB) ^ (4 * (rr & 3))) * 8;
                if (x > a.J - 8) x = a.J - 8;
                goff[q] = rr * a.B.ld + x;
            } else {
                int64_t j = n0 + (trow - BM);
                if (j >= a.J) j = a.J - 1;
                goff[q] = row_offset(a.B, sv, j) + chunk * 8;
            }
        }
    }
    // Operands whose reduction columns are gathered by sample (the
    // per-sample transposed pool of the weight-gradient GEMM): lane q of
    // every wave holds the base offset of sample segment q of this step,
    // read back with v_readlane, and an issue cursor advances through the
    // segments by BK, so the loop neither divides nor waits on a table load.
    // (More than 64 segments fall back to the direct lookup.)
    const bool scA = a.A.seg_len > 0 && a.A.seg_cols, scB = a.B.seg_len > 0 && a.B.seg_cols;
    const int64_t nsegA = scA ? a.R / a.A.seg_len : 0, nsegB = scB ? a.R / a.B.seg_len : 0;
    const bool fastA = nsegA <= 64, fastB = nsegB <= 64;
    int64_t segvA = 0, segvB = 0;
    if (scA && fastA && lane < nsegA) segvA = sv.id(lane) * a.A.seg_stride;
    if (scB && fastB && lane < nsegB) segvB = sv.id(lane) * a.B.seg_stride;
    auto lane_value = [](int64_t v, int32_t q) {
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, q);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)v >> 32), q);
        return (int64_t)(((uint64_t)hi << 32) | lo);
    };
    int64_t kq = 0;                 // reduction column of the next issue
    int32_t segA = 0, offA = 0, segB = 0, offB = 0;
    auto issue = [&](StageMem st) {
        int64_t ca = kq, cb = kq;
        if (scA) {
            ca = fastA ? lane_value(segvA, segA) + offA : col_offset(a.A, sv, kq);
            offA += BK;
            if (offA == a.A.seg_len) { offA = 0; ++segA; }
        }
        if (scB) {
            cb = fastB ? lane_value(segvB, segB) + offB : col_offset(a.B, sv, kq);
            offB += BK;
            if (offB == a.B.seg_len) { offB = 0; ++segB; }
        }
        if constexpr (AT) ca = kq * a.A.ld;
        if constexpr (BT) cb = kq * a.B.ld;
        kq += BK;
        static_for<LPW>([&](auto Qi) {
            constexpr int q = decltype(Qi)::value;
            const int p = wave + q * NW;
            if constexpr (q < QA) {
                __builtin_amdgcn_global_load_lds((gbl_void*)(Ab + ca + goff[q]), (lds_void*)(st.A + p * RPL * ROWB),
                                                 16, 0, 0);
            } else {
                __builtin_amdgcn_global_load_lds((gbl_void*)(Bb + cb + goff[q]),
                                                 (lds_void*)(st.B + (p * RPL - BM) * ROWB), 16, 0, 0);
            }
        });
    };

    floatx16 acc[TM][TN];
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[tm][tn][r] = 0.0f;

    const int64_t nk = Rk / BK;
    static_for<STAGES - 1>([&](auto I) {
        if (decltype(I)::value < nk) issue(stage_mem(I));
    });

    const int frow = lane & 31, fhalf = lane >> 5;
    for (int64_t kb = 0; kb < nk; kb += STAGES) {
        static_for<STAGES>([&](auto I) {
            constexpr int st = decltype(I)::value;
            const int64_t kt = kb + st;
            if (kt >= nk) return;
            // stage kt complete for this wave; later stages may stay in flight
            const int64_t ahead = (nk - 1 - kt) < (STAGES - 2) ? (nk - 1 - kt) : (STAGES - 2);
            wait_vmcnt_upto<LPW, STAGES - 2>((int)ahead);
            lds_barrier();
            if (kt + STAGES - 1 < nk) issue(stage_mem(std::integral_constant<int, (st + STAGES - 1) % STAGES>{}));
            const char* As = stage_mem(I).A;
            const char* Bs = stage_mem(I).B;
            constexpr int KS = BK / 16;
            bf16x8 af[KS][TM], bfr[KS][TN];
            auto frag = [&](const char* base, int row, int c) {
                return *reinterpret_cast<const bf16x8*>(base + row * ROWB + ((c ^ ((row / RPW) % SLOTS)) << 4));
            };
            // Fragment of a transposed operand: lane l needs reduction rows
            // 16 ks + 8 (l / 32) + 0..7 of output index col0 + l % 32.
            // ds_read_b64_tr_b16 gives lane i of a 16-lane group element i % 4
            // of the 8-byte piece addressed by lane 4 e + i / 4, for e = 0..3;
            // so lane s addresses row rowb + s / 4 at output index
            // colb + 4 (s % 4), and lane i receives rows rowb + e of index
            // colb + i.  Two reads cover the 8 rows.
            auto fragT = [&](const char* base, auto RT, int col0, int ks) {
                constexpr int ROWT = decltype(RT)::value;
                typedef short v4s __attribute__((ext_vector_type(4)));
                typedef short v8s __attribute__((ext_vector_type(8)));
                const int g = lane >> 4, sl = lane & 15;
                const int r = ks * 16 + 8 * (g >> 1) + (sl >> 2);
                const int x = col0 + 16 * (g & 1) + 4 * (sl & 3);
                const char* p0 = base + r * ROWT + (((x >> 3) ^ (4 * (r & 3))) << 4) + (x & 7) * 2;
                const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p0));
                const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p0 + 4 * ROWT));
                const v8s v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                return __builtin_bit_cast(bf16x8, v);
            };
            auto load_sub = [&](int ks) {
#pragma unroll
                for (int tm = 0; tm < TM; ++tm) {
                    if constexpr (AT)
                        af[ks][tm] = fragT(As, std::integral_constant<int, ROWTA>{}, wm * WM + tm * 32, ks);
                    else
                        af[ks][tm] = frag(As, wm * WM + tm * 32 + frow, ks * 2 + fhalf);
                }
#pragma unroll
                for (int tn = 0; tn < TN; ++tn) {
                    if constexpr (BT)
                        bfr[ks][tn] = fragT(Bs, std::integral_constant<int, ROWTB>{}, wn * WN + tn * 32, ks);
                    else
                        bfr[ks][tn] = frag(Bs, wn * WN + tn * 32 + frow, ks * 2 + fhalf);
                }
            };
#pragma unroll
            for (int ks = 0; ks < KPRE; ++ks) load_sub(ks);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                for (int tm = 0; tm < TM; ++tm)
#pragma unroll
                    for (int tn = 0; tn < TN; ++tn)
                        acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks][tm], bfr[ks][tn], acc[tm][tn], 0, 0, 0);
                if (ks + KPRE < KS) load_sub(ks + KPRE);
                // let the scheduler interleave this sub-step's MFMAs with the
                // next sub-step's fragment reads (LLVM's MFMA/DS-read
                // interleaving strategy 1); the arithmetic is unchanged
                __builtin_amdgcn_iglp_opt(1);
            }
        });
    }

    if constexpr (EPI == EPI_STE) {
        double L = 0.0;
        if (folded) {
            L = fold_decide(a, stv, fold_pre);
            if (!__builtin_isfinite(L)) {   // the loop stops: no update
                fold_arrive(a, L);
                return;
            }
        }
        if constexpr (RING) {
            epilogue_ste_ring<BM, BN, NT, WM, WN, TM, TN, ABYTES, GL, CHUNK_TIES>(a, stv, acc, m0, n0, wm, wn, lane, sa0,
                                                                                 sb0, sa1,
                                                                  sb1);
        } else {
            epilogue_ste<BM, BN, NT, WM, WN, TM, TN, ABYTES>(a, stv, acc, m0, n0, wm, wn, lane, sa0);
        }
        if (folded) fold_arrive(a, L);
    } else {
        epilogue_lds<BM, BN, NT, WM, WN, TM, TN, EPI, ABYTES>(a, sv, acc, m0, n0, wm, wn, lane, sa0,
                                                                           red, out);
        if (EPI == EPI_LOSS) {
            __syncthreads();
            if (tid == 0) {
                double s = 0.0;
                for (int w = 0; w < NW; ++w) s += red[w];
                a.partials[blockIdx.x] = s;
            }
        }
    }
}

// LDS of the fused-epilogue instantiation (its DMA ring reuses the stages).
constexpr int ste_lds_bytes(int BM, int BN, int BK, int NW, int STAGES) {
    return STAGES * (BM + BN) * BK * 2;
}

template <int BM, int BN, int BK, int NWM, int NWN, int STAGES, int KPRE = BK / 16, bool AT = false, bool BT = false>
hipError_t launch_bf16_dma(const GemmArgs& a, int32_t* nb, hipStream_t stream) {
    const int64_t tiles = ((a.I + BM - 1) / BM) * ((a.J + BN - 1) / BN);
    if constexpr (AT || BT) {
        if (a.epi != EPI_STORE) return hipErrorInvalidValue;
        hipLaunchKernelGGL((gemm_bf16_dma_kernel<BM, BN, BK, NWM, NWN, STAGES, EPI_STORE, KPRE, false, false, AT, BT>),
                           dim3((unsigned)tiles), dim3(NWM * NWN * 64), 0, stream, a);
        if (nb) *nb = (int32_t)tiles;
        return hipGetLastError();
    }
    if (a.epi == EPI_LOSS)
        hipLaunchKernelGGL((gemm_bf16_dma_kernel<BM, BN, BK, NWM, NWN, STAGES, EPI_LOSS, KPRE>), dim3((unsigned)tiles),
                           dim3(NWM * NWN * 64), 0, stream, a);
    else if (a.epi == EPI_STE) {
        if constexpr (ste_lds_bytes(BM, BN, BK, NWM * NWN, STAGES) <= 160 * 1024 &&
                      rows_per_pass(BM, BN, BM * BK * 2) > 0) {
            // Asymmetric g128 and g32 (the layer and decoder workloads) get
            // epilogues specialised on the group size.  The near-tie tests
            // share one branch per chunk when the grid runs several rounds of
            // tiles (MLP block 1.872 -> 1.850 ms, 7B block 3.344 -> 3.311 ms,
            // 70B block 7.59 -> 7.44 ms per step) and keep one per weight when
            // every CU takes a single tile (the 4096 x 4096 layer, 0.5 us
            // faster that way).
            const int gl = a.fu.qp.sym ? 0 : a.fu.qp.group / 8;
            const bool rounds = tiles > 256;
            if (a.fu.w_bf16 && gl == 16 && rounds)
                hipLaunchKernelGGL(
                    (gemm_bf16_dma_kernel<BM, BN, BK, NWM, NWN, STAGES, EPI_STE, KPRE, true, false, false, false, 16, true>),
                    dim3((unsigned)tiles), dim3(NWM * NWN * 64), 0, stream, a);
            else if (a.fu.w_bf16 && gl == 16)
                hipLaunchKernelGGL(
                    (gemm_bf16_dma_kernel<BM, BN, BK, NWM, NWN, STAGES, EPI_STE, KPRE, true, false, false, false, 16>),
                    dim3((unsigned)tiles), dim3(NWM * NWN * 64), 0, stream, a);
            else if (a.fu.w_bf16 && gl == 4)
                hipLaunchKernelGGL(
                    (gemm_bf16_dma_kernel<BM, BN, BK, NWM, NWN, STAGES, EPI_STE, KPRE, true, false, false, false, 4, true>),
                    dim3((unsigned)tiles), dim3(NWM * NWN * 64), 0, stream, a);
            else if (a.fu.w_bf16)
                hipLaunchKernelGGL((gemm_bf16_dma_kernel<BM, BN, BK, NWM, NWN, STAGES, EPI_STE, KPRE, true>),
                                   dim3((unsigned)tiles), dim3(NWM * NWN * 64), 0, stream, a);
            else
                hipLaunchKernelGGL((gemm_bf16_dma_kernel<BM, BN, BK, NWM, NWN, STAGES, EPI_STE, KPRE, false>),
                                   dim3((unsigned)tiles), dim3(NWM * NWN * 64), 0, stream, a);
        }
        else
            return hipErrorInvalidValue;
    }
    else
        hipLaunchKernelGGL((gemm_bf16_dma_kernel<BM, BN, BK, NWM, NWN, STAGES, EPI_STORE, KPRE>), dim3((unsigned)tiles),
                           dim3(NWM * NWN * 64), 0, stream, a);
    if (nb) *nb = (int32_t)tiles;
    return hipGetLastError();
}

// Launch one bf16 configuration; returns the workgroup count through *nb.
template <int BM, int BN, int BK, int NWM, int NWN>
hipError_t launch_bf16(const GemmArgs& a, int32_t* nb, hipStream_t stream) {
    const int64_t tiles = ((a.I + BM - 1) / BM) * ((a.J + BN - 1) / BN);
    if (a.epi == EPI_LOSS)
        hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, BK, NWM, NWN, EPI_LOSS>), dim3((unsigned)tiles),
                           dim3(NWM * NWN * 64), 0, stream, a);
    else
        hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, BK, NWM, NWN, EPI_STORE>), dim3((unsigned)tiles),
                           dim3(NWM * NWN * 64), 0, stream, a);
    if (nb) *nb = (int32_t)tiles;
    return hipGetLastError();
}

template <int BM, int BN, int BK, int NWM, int NWN>
hipError_t launch_f32(const GemmArgs& a, int32_t* nb, hipStream_t stream) {
    const int64_t tiles = ((a.I + BM - 1) / BM) * ((a.J + BN - 1) / BN);
    if (a.epi == EPI_LOSS)
        hipLaunchKernelGGL((gemm_f32_kernel<BM, BN, BK, NWM, NWN, EPI_LOSS>), dim3((unsigned)tiles),
                           dim3(NWM * NWN * 64), 0, stream, a);
    else
        hipLaunchKernelGGL((gemm_f32_kernel<BM, BN, BK, NWM, NWN, EPI_STORE>), dim3((unsigned)tiles),
                           dim3(NWM * NWN * 64), 0, stream, a);
    if (nb) *nb = (int32_t)tiles;
    return hipGetLastError();
}

}  // namespace gemm
}  // namespace ar
