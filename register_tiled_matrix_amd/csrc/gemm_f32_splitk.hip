// gemm_f32_splitk.hip -- the fp32 register-tiled kernel for problems with few output tiles
// (tall-skinny or small M, N): split-K inside the workgroup.
//
// With 128x128 tiles a 16384 x 128 output is only 128 workgroups for 256 CUs, half a wave per
// SIMD. Here a workgroup owns a 64x64 tile and each of its four waves accumulates that whole
// tile over its own quarter of K, with the same register micro-tile as the square kernel
// ("Understanding Register Tiling" (blog.csdn.net/sweet_ran), the key loop: regA[8],
// regB[8], 64 FMAs per k held in registers; "寄存器Tiling跨架构解析" section 2.4 / 7.2: trade
// tile size against the number of resident waves). The four partial tiles are then summed
// through LDS in a fixed order (wave 0 + wave 1 + wave 2 + wave 3), so results are
// deterministic; the summation order differs from the square kernel's single k sweep.
//
// Per wave: 64 lanes as an 8x8 grid, lane micro-tile rows {r0..r0+3, r0+32..r0+35} and columns
// {c0..c0+3, c0+32..c0+35} (every wave-wide 16-byte fragment read is one contiguous 128-byte
// run). Each wave stages its own A slab (k-major, padded) and B slab in LDS, double-buffered;
// the workgroup still synchronises once per slab.
#include "regtile_internal.h"

namespace regtile {

namespace {

constexpr int TILE = 64, NW = 4, NT = 256, BK = 16, APAD = 4;
constexpr int AS = TILE + APAD;  // A slab row stride (floats), k-major

struct alignas(16) WaveStage {
    float a[BK][AS];
    float b[BK][TILE];
};
struct alignas(16) Smem {
    union {
        WaveStage st[NW][2];
        float part[NW][TILE][TILE + 4];  // the four partial tiles after the main loop (padded)
    };
};

template <bool GUARD, bool VEC>
__device__ __forceinline__ float4 load4(const float *__restrict__ p, bool row_ok, int cols_left) {
    if (!GUARD) {
        if (VEC) return *reinterpret_cast<const float4 *>(p);
        return make_float4(p[0], p[1], p[2], p[3]);
    }
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (row_ok) {
        if (VEC && cols_left >= 4) {
            v = *reinterpret_cast<const float4 *>(p);
        } else {
            if (cols_left > 0) v.x = p[0];
            if (cols_left > 1) v.y = p[1];
            if (cols_left > 2) v.z = p[2];
            if (cols_left > 3) v.w = p[3];
        }
    }
    return v;
}

// GUARD: bounds checks on every load (ragged M/N, or K not a multiple of 4*BK).
template <bool GUARD, bool VEC_A, bool VEC_B, bool VEC_C>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2))) void f32_splitk_kernel(
    int M, int N, int K, float alpha, const float *__restrict__ A, int64_t lda,
    const float *__restrict__ B, int64_t ldb, float beta, float *__restrict__ C, int64_t ldc,
    int tiles_m, int tiles_n, int slabs_per_wave) {
    __shared__ Smem sm;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r0 = (lane >> 3) * 4, c0 = (lane & 7) * 4;

    int tm, tn;
    grouped_tile<8>(xcd_contiguous_id(blockIdx.x, gridDim.x), tiles_m, tiles_n, tm, tn);
    const int m0 = tm * TILE, n0 = tn * TILE;
    const int kb = wave * slabs_per_wave * BK;           // this wave's k range [kb, ke)
    const int ke = min(K, kb + slabs_per_wave * BK);

    // Staging: A slab 64 rows x 16 k = 256 float4 -> 4 per lane (row q/4, k (q%4)*4);
    //          B slab 16 k x 64 cols  = 256 float4 -> 4 per lane (k q/16, col (q%16)*4).
    float4 ra[4], rb[4];
    auto load_slab = [&](int k0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = lane + 64 * i;
            const int ar = q >> 2, ak = (q & 3) * 4;
            ra[i] = load4<GUARD, VEC_A>(A + (int64_t)(m0 + ar) * lda + k0 + ak, m0 + ar < M,
                                        ke - (k0 + ak));
            const int bk = q >> 4, bc = (q & 15) * 4;
            rb[i] = load4<GUARD, VEC_B>(B + (int64_t)(k0 + bk) * ldb + n0 + bc, k0 + bk < ke,
                                        N - (n0 + bc));
        }
    };
    auto store_slab = [&](int buf) {
        WaveStage &w = sm.st[wave][buf];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = lane + 64 * i;
            const int ar = q >> 2, ak = (q & 3) * 4;
            w.a[ak + 0][ar] = ra[i].x;
            w.a[ak + 1][ar] = ra[i].y;
            w.a[ak + 2][ar] = ra[i].z;
            w.a[ak + 3][ar] = ra[i].w;
            const int bk = q >> 4, bc = (q & 15) * 4;
            *reinterpret_cast<float4 *>(&w.b[bk][bc]) = rb[i];
        }
    };

    float acc[8][8];
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int n = 0; n < 8; ++n) acc[m][n] = 0.0f;

    auto compute_slab = [&](int buf) {
        const float *sa = &sm.st[wave][buf].a[0][0] + r0;
        const float *sb = &sm.st[wave][buf].b[0][0] + c0;
        float4 fa[2][2], fb[2][2];
        fa[0][0] = *reinterpret_cast<const float4 *>(sa);
        fa[0][1] = *reinterpret_cast<const float4 *>(sa + 32);
        fb[0][0] = *reinterpret_cast<const float4 *>(sb);
        fb[0][1] = *reinterpret_cast<const float4 *>(sb + 32);
#pragma unroll
        for (int k = 0; k < BK; ++k) {
            const int cb = k & 1, nb = cb ^ 1;
            if (k + 1 < BK) {
                fa[nb][0] = *reinterpret_cast<const float4 *>(sa + (k + 1) * AS);
                fa[nb][1] = *reinterpret_cast<const float4 *>(sa + (k + 1) * AS + 32);
                fb[nb][0] = *reinterpret_cast<const float4 *>(sb + (k + 1) * TILE);
                fb[nb][1] = *reinterpret_cast<const float4 *>(sb + (k + 1) * TILE + 32);
            }
            const float a_[8] = {fa[cb][0].x, fa[cb][0].y, fa[cb][0].z, fa[cb][0].w,
                                 fa[cb][1].x, fa[cb][1].y, fa[cb][1].z, fa[cb][1].w};
            const float b_[8] = {fb[cb][0].x, fb[cb][0].y, fb[cb][0].z, fb[cb][0].w,
                                 fb[cb][1].x, fb[cb][1].y, fb[cb][1].z, fb[cb][1].w};
#pragma unroll
            for (int m = 0; m < 8; ++m)
#pragma unroll
                for (int n = 0; n < 8; ++n) acc[m][n] = fmaf(a_[m], b_[n], acc[m][n]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Every wave runs the same number of slabs (barrier counts must match); a wave whose
    // range is shorter loads zeros past ke.
    if (slabs_per_wave > 0) {
        load_slab(kb);
        store_slab(0);
        __syncthreads();
        for (int s = 0; s + 1 < slabs_per_wave; ++s) {
            load_slab(kb + (s + 1) * BK);
            compute_slab(s & 1);
            store_slab((s + 1) & 1);
            __syncthreads();
        }
        compute_slab((slabs_per_wave - 1) & 1);
    }
    __syncthreads();  // all waves are done with their stages: the union turns into partials

    // Partial tile of this wave -> LDS.
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const int row = r0 + (m < 4 ? m : 28 + m);
        *reinterpret_cast<float4 *>(&sm.part[wave][row][c0]) =
            make_float4(acc[m][0], acc[m][1], acc[m][2], acc[m][3]);
        *reinterpret_cast<float4 *>(&sm.part[wave][row][c0 + 32]) =
            make_float4(acc[m][4], acc[m][5], acc[m][6], acc[m][7]);
    }
    __syncthreads();

    // Fixed-order sum and epilogue: thread t owns row t/4, columns (t%4)*16 .. +15.
    const int row = tid >> 2, col0 = (tid & 3) * 16;
    const int grow = m0 + row;
    if (GUARD && grow >= M) return;
    float *crow = C + (int64_t)grow * ldc;
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) {
        const int col = col0 + c4 * 4;
        float4 s = *reinterpret_cast<const float4 *>(&sm.part[0][row][col]);
#pragma unroll
        for (int w = 1; w < NW; ++w) {
            const float4 p = *reinterpret_cast<const float4 *>(&sm.part[w][row][col]);
            s.x += p.x;
            s.y += p.y;
            s.z += p.z;
            s.w += p.w;
        }
        const int gcol = n0 + col;
        float *c = crow + gcol;
        if (VEC_C && (!GUARD || gcol + 3 < N)) {
            float4 v;
            if (beta == 0.0f) {
                v = make_float4(alpha * s.x, alpha * s.y, alpha * s.z, alpha * s.w);
            } else {
                const float4 old = *reinterpret_cast<const float4 *>(c);
                v = make_float4(fmaf(alpha, s.x, beta * old.x), fmaf(alpha, s.y, beta * old.y),
                                fmaf(alpha, s.z, beta * old.z), fmaf(alpha, s.w, beta * old.w));
            }
            *reinterpret_cast<float4 *>(c) = v;
        } else {
            const float sv[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (!GUARD || gcol + e < N) c[e] = epilogue_value(sv[e], alpha, beta, c + e);
        }
    }
}

template <bool G, bool VA, bool VB, bool VC>
hipError_t launch_variant(const Problem &p, hipStream_t s, int tm, int tn, int spw) {
    hipLaunchKernelGGL((f32_splitk_kernel<G, VA, VB, VC>), dim3(tm * tn), dim3(NT), 0, s, p.M, p.N,
                       p.K, p.alpha, (const float *)p.A, p.lda, (const float *)p.B, p.ldb, p.beta,
                       p.C, p.ldc, tm, tn, spw);
    return hipGetLastError();
}
template <bool G, bool VA, bool VB>
hipError_t pick_c(const Problem &p, hipStream_t s, int tm, int tn, int spw, bool vc) {
    return vc ? launch_variant<G, VA, VB, true>(p, s, tm, tn, spw)
              : launch_variant<G, VA, VB, false>(p, s, tm, tn, spw);
}
template <bool G, bool VA>
hipError_t pick_b(const Problem &p, hipStream_t s, int tm, int tn, int spw, bool vb, bool vc) {
    return vb ? pick_c<G, VA, true>(p, s, tm, tn, spw, vc) : pick_c<G, VA, false>(p, s, tm, tn, spw, vc);
}
template <bool G>
hipError_t pick_a(const Problem &p, hipStream_t s, int tm, int tn, int spw, bool va, bool vb, bool vc) {
    return va ? pick_b<G, true>(p, s, tm, tn, spw, vb, vc) : pick_b<G, false>(p, s, tm, tn, spw, vb, vc);
}


}  // namespace

hipError_t launch_f32_splitk(const Problem &p, hipStream_t s, const char **name) {
    const int tiles_m = (p.M + TILE - 1) / TILE, tiles_n = (p.N + TILE - 1) / TILE;
    const int nslabs = (p.K + BK - 1) / BK;
    const int spw = (nslabs + NW - 1) / NW;  // slabs per wave
    const bool guard = (p.M % TILE) != 0 || (p.N % TILE) != 0 || (p.K % (NW * BK)) != 0;
    const bool va = (p.lda % 4) == 0 && aligned16(p.A);
    const bool vb = (p.ldb % 4) == 0 && aligned16(p.B);
    const bool vc = (p.ldc % 4) == 0 && aligned16(p.C);
    *name = guard ? "f32_regtile_splitk4_64x64x16_8x8_guard" : "f32_regtile_splitk4_64x64x16_8x8";
    return guard ? pick_a<true>(p, s, tiles_m, tiles_n, spw, va, vb, vc)
                 : pick_a<false>(p, s, tiles_m, tiles_n, spw, va, vb, vc);
}

}  // namespace regtile
