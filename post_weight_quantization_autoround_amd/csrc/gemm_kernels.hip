// MFMA GEMMs of the tuning loop (gfx950).
//
// Both GEMMs of a step (blog sec. 3 algorithm flow: the QDQ forward and the
// back-propagation) are written as C[i, j] = sum_r A[i, r] * B[j, r] with
// both operands contiguous along the reduction index r:
//   forward  Y^T[n, m] = sum_k w^[n, k] * X_b[m, k]     (A = w^, B = X_b)
//   wgrad    G[n, k]   = sum_m dY^T[n, m] * X_b^T[k, m] (A = dY^T, B = X_b^T)
// The reference output is kept per sample as [S, N, T] so the forward
// epilogue reads it and writes dY^T along contiguous columns, and the pool
// is kept transposed per sample ([S, K, T]) in HBM, so neither GEMM needs a
// transpose in LDS.  Rows of X_b (forward) and reduction columns of X_b^T (wgrad) are
// gathered from the pool by a per-step sample table in device memory, so one
// captured launch serves every step.

#include "gemm_tiles.h"

namespace ar {

using namespace gemm;

namespace {

// Tile choice (bf16, measured on MI355X for the 4096 x 4096 layer with 2048
// tokens per step).  Loss GEMM (rows n, columns m): 256 x 128 tiles with
// eight wavefronts and three LDS stages when that still gives one tile per
// CU, else 128 x 128 (two workgroups per CU).  Other GEMMs: 256 x 256 tiles
// with eight wavefronts when the grid has at least one per CU, else
// 128 x 128.  Reduction lengths that are multiples of 64 (with a column count
// that is a multiple of 8) take the LDS-direct kernels, others the
// register-staged ones.
enum Plan { P128_DMA, P256_DMA, P256x128_DMA, P128_REG, P256_REG };

Plan plan_bf16(const GemmArgs& a) {
    const bool dma = (a.R % 64) == 0 && (a.J % 8) == 0 && (!a.A.trans || a.I % 8 == 0);
    if (a.epi == EPI_LOSS) {
        const bool tall = ((a.I + 255) / 256) * ((a.J + 127) / 128) >= 256;
        if (dma) return tall ? P256x128_DMA : P128_DMA;
        return P128_REG;
    }
    const bool wide = ((a.I + 255) / 256) * ((a.J + 255) / 256) >= 256;
    if (wide) return dma ? P256_DMA : P256_REG;
    return dma ? P128_DMA : P128_REG;
}

void plan_tile(Plan p, int64_t& bm, int64_t& bn) {
    switch (p) {
        case P256_DMA: case P256_REG: bm = 256; bn = 256; break;
        case P256x128_DMA: bm = 256; bn = 128; break;
        default: bm = 128; bn = 128; break;
    }
}

// One DMA configuration with the operands' storage order (a transposed
// operand only in plain-store GEMMs, checked by the caller).  A transposed
// B operand swaps the wavefront grid (NWN x NWM): each of its fragments
// costs two ds_read_b64_tr_b16, so wavefronts that span fewer B columns
// read fewer of them (70B dh2: 1.05 -> 0.91 ms).
template <int BM, int BN, int BK, int NWM, int NWN, int STAGES, int KPRE>
hipError_t launch_dma(const GemmArgs& a, int32_t* nb, hipStream_t stream) {
    if (a.A.trans) return launch_bf16_dma<BM, BN, BK, NWM, NWN, STAGES, KPRE, true, false>(a, nb, stream);
    if (a.B.trans) return launch_bf16_dma<BM, BN, BK, NWN, NWM, STAGES, KPRE, false, true>(a, nb, stream);
    return launch_bf16_dma<BM, BN, BK, NWM, NWN, STAGES, KPRE>(a, nb, stream);
}

}  // namespace

int32_t gemm_grid_blocks(bool bf16, int64_t I, int64_t J, int64_t R, int epi) {
    if (bf16) {
        GemmArgs a{};
        a.I = I; a.J = J; a.R = R; a.epi = epi;
        int64_t bm, bn;
        plan_tile(plan_bf16(a), bm, bn);
        return (int32_t)(((I + bm - 1) / bm) * ((J + bn - 1) / bn));
    }
    return (int32_t)(((I + 127) / 128) * ((J + 127) / 128));
}

int32_t gemm_fused_tile_cols(int64_t I, int64_t J, int64_t R) {
    GemmArgs a{};
    a.I = I; a.J = J; a.R = R; a.epi = EPI_STE;
    switch (plan_bf16(a)) {
        case P256_DMA: return 256;
        case P128_DMA: return 128;
        default: return 0;
    }
}

namespace {

// A plain-store grid of 256 x 256 tiles a little over a whole number of
// rounds of the 256 CUs would spend its last round on a few tiles while most
// CUs idle (the MLP's dH GEMM: 344 tiles, 1.34 rounds, 2 rounds of time).
// Then the whole rounds run as 256 x 256 tiles and the remaining rows (or
// columns) as 256 x 128 tiles, twice as many of half the work, in a second
// launch that fits one round.  Only an operand that is not gathered by
// sample is split, so its rows can be offset directly.
bool launch_split_tail(const GemmArgs& a, int32_t* nblocks, hipStream_t stream, hipError_t* err) {
    if (a.epi != EPI_STORE) return false;
    const int64_t tm = (a.I + 255) / 256, tn = (a.J + 255) / 256, tiles = tm * tn;
    const int64_t full = (tiles / 256) * 256, rest = tiles - full;
    if (full == 0 || rest == 0 || 2 * rest > 256) return false;
    GemmArgs a1 = a, a2 = a;
    if (a.A.seg_len == 0 && full % tn == 0) {
        const int64_t i1 = (full / tn) * 256;
        a1.I = i1;
        a2.I = a.I - i1;
        a2.A.base = static_cast<const uint16_t*>(a.A.base) + (a.A.trans ? i1 : i1 * a.A.ld);
        a2.out = a.out + i1 * a.ldc;
    } else if (a.B.seg_len == 0 && full % tm == 0) {
        const int64_t j1 = (full / tm) * 256;
        a1.J = j1;
        a2.J = a.J - j1;
        a2.B.base = static_cast<const uint16_t*>(a.B.base) + (a.B.trans ? j1 : j1 * a.B.ld);
        a2.out = a.out + j1;
    } else {
        return false;
    }
    int32_t n1 = 0, n2 = 0;
    *err = launch_dma<256, 256, 64, 4, 2, 2, 1>(a1, &n1, stream);
    if (*err == hipSuccess) *err = launch_dma<256, 128, 64, 4, 2, 3, 2>(a2, &n2, stream);
    if (nblocks) *nblocks = n1 + n2;
    return true;
}

}  // namespace

// A transposed operand: plain store, unsegmented, at most one of the two,
// at least 8 output indices along it (its loads are clamped to the last
// 16-byte chunk) and the reduction a multiple of 64 (the DMA kernels).
bool trans_ok(const GemmArgs& a) {
    if (!a.A.trans && !a.B.trans) return true;
    if (a.A.trans && a.B.trans) return false;
    if (a.epi != EPI_STORE || a.R % 64 != 0 || a.J % 8 != 0) return false;
    if (a.A.trans && (a.A.seg_len != 0 || a.I % 8 != 0 || a.A.ld < a.I)) return false;
    if (a.B.trans && (a.B.seg_len != 0 || a.B.ld < a.J)) return false;
    return true;
}

hipError_t launch_gemm_bf16(const GemmArgs& a, int32_t* nblocks, hipStream_t stream) {
    if (a.epi == EPI_STE && gemm_fused_tile_cols(a.I, a.J, a.R) == 0) return hipErrorInvalidValue;
    if (a.out2 != nullptr) return hipErrorInvalidValue;   // split launches go through launch_gemm_bf16_split2
    if (!trans_ok(a)) return hipErrorInvalidValue;
    if (plan_bf16(a) == P256_DMA) {
        hipError_t e = hipSuccess;
        if (launch_split_tail(a, nblocks, stream, &e)) return e;
    }
    switch (plan_bf16(a)) {
        case P256_DMA: return launch_dma<256, 256, 64, 4, 2, 2, 1>(a, nblocks, stream);
        case P256x128_DMA: return launch_dma<256, 128, 64, 4, 2, 3, 2>(a, nblocks, stream);
        case P128_DMA: return launch_dma<128, 128, 64, 2, 2, 2, 1>(a, nblocks, stream);
        case P256_REG: return launch_bf16<256, 256, 64, 2, 4>(a, nblocks, stream);
        default: return launch_bf16<128, 128, 64, 2, 2>(a, nblocks, stream);
    }
}

bool gemm_split2_fits(const GemmArgs& a) {
    const int64_t tiles = ((a.I + 255) / 256) * ((a.J + 255) / 256);
    return a.epi == EPI_STORE && a.A.seg_len == 0 && a.B.seg_len == 0 && a.R % 128 == 0 && a.J % 8 == 0 &&
           a.R >= 4096 && 2 * tiles <= 256 && 2 * tiles > 192 && !a.A.trans && trans_ok(a);
}

hipError_t launch_gemm_bf16_split2(const GemmArgs& a, hipStream_t stream) {
    if (!gemm_split2_fits(a) || a.out2 == nullptr) return hipErrorInvalidValue;
    const int64_t tiles = ((a.I + 255) / 256) * ((a.J + 255) / 256);
    if (a.B.trans)
        hipLaunchKernelGGL((gemm_bf16_dma_kernel<256, 256, 64, 2, 4, 2, EPI_STORE, 1, false, true, false, true>),
                           dim3((unsigned)tiles, 2), dim3(512), 0, stream, a);
    else
        hipLaunchKernelGGL((gemm_bf16_dma_kernel<256, 256, 64, 4, 2, 2, EPI_STORE, 1, false, true>),
                           dim3((unsigned)tiles, 2), dim3(512), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_gemm_f32(const GemmArgs& a, int32_t* nblocks, hipStream_t stream) {
    return launch_f32<128, 128, 32, 2, 2>(a, nblocks, stream);
}

}  // namespace ar
