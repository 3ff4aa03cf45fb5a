// ssd_bf16.hip -- gfx950 state-pass and chunk-output kernels for bf16 inputs
// (bf16 MFMA operands, fp32 accumulation, fp32 running state).
//
// Method: dbyun.net, "基于 NVIDIA CUDA Tile 加速 Mamba-2 高性能前向传播内核",
// sections "Kernel 2: fwd_pass_state" (decayed chunk jump) and
// "Kernel 3：compute_out" (decayed chunk output).
//
// Both kernels contract over tokens, which are the strided dimension of every
// input tensor.  Tiles are copied into LDS in their natural token-major layout
// with 16-byte writes and the token-packed MFMA operands are read back with
// the gfx950 LDS transpose read (ds_read_b64_tr_b16), so no element-wise
// transposition happens on the way in.
#include <algorithm>

#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

__device__ __forceinline__ bf16x8 ld16(const bf16 *p) { return *reinterpret_cast<const bf16x8 *>(p); }

__device__ __forceinline__ bf16x8 zero8()
{
    bf16x8 z;
#pragma unroll
    for (int e = 0; e < 8; ++e) z[e] = (bf16)0.0f;
    return z;
}

// WG index -> (major, minor) with all minors of one major on the same XCD when
// `xcd` is set (workgroups are dealt to the 8 XCDs round-robin by index).
__device__ __forceinline__ void xcd_split(int id, int n_minor, bool xcd, int &major, int &minor)
{
    if (xcd) {
        const int x = id & 7, slot = id >> 3;
        major = x + 8 * (slot / n_minor);
        minor = slot % n_minor;
    } else {
        major = id / n_minor;
        minor = id % n_minor;
    }
}

// ===========================================================================
// State pass.  Workgroup = one (batch*head, N tile of NT columns, group of up
// to K consecutive chunks).  It keeps h^T [NT x 64] in fp32 accumulators: wave
// (ph, nh, kh) owns rows n in [32 nh, 32 nh + 32) and columns p in
// [32 ph, 32 ph + 32) for the tokens of K-half kh (KS = 2 splits each chunk's
// tokens over two wave sets whose partial states are summed through LDS at
// every chunk boundary).
//
// Groups.  The chunk jump h <- a_c h + U_c is linear, so a run of chunks can
// start from a zero state and be corrected afterwards: group g (chunks
// [gK, gK+K)) starts from h0 if g == 0 and from 0 otherwise, stores its local
// chunk-start states, its final local state U_g, the decay products
// beta_c = prod_{gK <= c' < c} a_c' and gamma_g = prod_{c' in g} a_c'.  A scan
// over groups (group_scan_kernel) then gives the true state at each group
// start, H_g, and the true chunk-start state is S_local[c] + beta_c H_g.  With
// one group (K >= nc) the kernel is the plain serial state pass and writes
// true states and hT directly.
//
// Operands, both k-packed by token:
//   * X (B operand): the x tile is copied into LDS as is, token-major [t][p],
//     with 16-byte writes of whole token rows, and read back with the LDS
//     transpose read;
//   * W (A operand): each thread loads an 8-token x WC-column block of B,
//     scales token t by its weight w_t (from stage 1) and bf16-packs the pairs
//     (t, t+1) of each column, which is already the k-packed layout WT[n][t];
//     read back as one 16-byte fragment per MFMA.
// The LDS tile is single-buffered (about 65 KB at Q = 256) so that two
// workgroups share a CU and overlap each other's loads, barriers and MFMAs;
// global loads still run two chunks ahead in registers.
// ===========================================================================
template <int Q, int NT, int KS>
__global__ __launch_bounds__(64 * 2 * (NT / 32) * KS) void state_pass_bf16_kernel(
    const bf16 *__restrict__ x, const bf16 *__restrict__ Bm, const float *__restrict__ G2,
    const float *__restrict__ wT, const float *__restrict__ h0, bf16 *__restrict__ S,
    float *__restrict__ hT, float *__restrict__ Ug, float *__restrict__ gam,
    float *__restrict__ beta, int L, int H, int G, int N, int nc, int Lp, int ntiles, int K,
    int ng, int xcd)
{
    constexpr int P = 64;
    constexpr int NWN = NT / 32, NWAVES = 2 * NWN * KS, NTHR = 64 * NWAVES;
    constexpr int KSTEPS = Q / 16 / KS;
    constexpr int XP = tr_pitch(P);                  // token-major x rows (elements)
    constexpr int PT = Q + 8;                        // k-packed W rows (elements)
    constexpr int XPC = Q * (P / 8) / NTHR;          // 16-byte x pieces per thread
    constexpr int WC = Q * NT / (8 * NTHR);          // W block: 8 tokens x WC columns
    constexpr int WD = (WC + 1) / 2;                 // dwords per loaded B row piece
    static_assert(XPC >= 1 && (Q * (P / 8)) % NTHR == 0, "x staging cover");
    static_assert(WC == 1 || WC == 2 || WC == 4 || WC == 8, "B staging block width");
    static_assert((Q / 8) * (NT / WC) == NTHR, "B staging cover");

    __shared__ __attribute__((aligned(16))) bf16 Xs[Q * XP];
    __shared__ __attribute__((aligned(16))) bf16 WT[NT * PT];
    __shared__ float red[KS > 1 ? (NWAVES / 2) * 16 * 64 : 1];
    __shared__ float alph;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ph = wave & 1, nh = (wave >> 1) % NWN, kh = wave / (2 * NWN);
    int bh, minor;
    xcd_split(blockIdx.x, ntiles * ng, xcd != 0, bh, minor);
    const int grp = minor / ntiles, nt = minor % ntiles;
    const int c0 = grp * K, c1 = min(c0 + K, nc);
    const int b = bh / H, h = bh % H, g = h / (H / G);
    const int n_wave = nt * NT + nh * 32;            // first state column of this wave's rows
    const int p_col = ph * 32 + (lane & 31);          // this lane's p
    const int n_lane = n_wave + 4 * (lane >> 5);      // + 8q + r for accumulator element 4q + r
    const int64_t st_off = (int64_t)bh * P * N;
    const float *Gh = G2 + (int64_t)bh * Lp;
    const float *wh = wT + (int64_t)bh * Lp;
    const int64_t xstride = (int64_t)H * P, bstride = (int64_t)G * N;
    const bf16 *xb = x + (int64_t)b * L * xstride + (int64_t)h * P;
    const bf16 *Bb = Bm + (int64_t)b * L * bstride + (int64_t)g * N + nt * NT;
    const bool keeper = nt == 0 && tid == 0;          // writes beta / gamma of this group

    f32x16 acc = zero_acc();
    if (h0 != nullptr && kh == 0 && grp == 0) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f32x4 v = *reinterpret_cast<const f32x4 *>(h0 + st_off + (int64_t)p_col * N + n_lane + 8 * q);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[4 * q + r] = v[r];
        }
    }

    // staging assignments: x piece r of this thread is token (tid + NTHR r) / 8,
    // p octet (tid + NTHR r) % 8; the B block is token group wtg, column group wcg
    int xo[XPC];
#pragma unroll
    for (int r = 0; r < XPC; ++r) {
        const int id = tid + NTHR * r;
        xo[r] = (id >> 3) * (int)xstride + (id & 7) * 8;
    }
    const int wtg = tid / (NT / WC), wcg = tid % (NT / WC);
    const int bo = wtg * 8 * (int)bstride + wcg * WC;

    struct Stage {
        bf16x8 xr[XPC];
        uint32_t br[8][WD];
        f32x4 w[2];
        float glast;
    };
    auto load_b_row = [&](uint32_t *dst, const bf16 *src) {
        if constexpr (WC == 8) {
            const u32x4 v = *reinterpret_cast<const u32x4 *>(src);
            dst[0] = v[0]; dst[1] = v[1]; dst[2] = v[2]; dst[3] = v[3];
        } else if constexpr (WC == 4) {
            const u32x2 v = *reinterpret_cast<const u32x2 *>(src);
            dst[0] = v[0]; dst[1] = v[1];
        } else if constexpr (WC == 2) {
            dst[0] = *reinterpret_cast<const uint32_t *>(src);
        } else {
            dst[0] = *reinterpret_cast<const uint16_t *>(src);
        }
    };
    auto issue = [&](Stage &st, int c) {
        const int t0 = c * Q;
        const bf16 *xc = xb + (int64_t)t0 * xstride;
        const bf16 *bc = Bb + (int64_t)t0 * bstride + bo;
        if (t0 + Q <= L) {   // full chunk (uniform): no per-lane predication
#pragma unroll
            for (int r = 0; r < XPC; ++r) st.xr[r] = ld16(xc + xo[r]);
#pragma unroll
            for (int r = 0; r < 8; ++r) load_b_row(st.br[r], bc + r * (int)bstride);
        } else {             // ragged last chunk: rows past L read as zero
#pragma unroll
            for (int r = 0; r < XPC; ++r) {
                const int t = (tid + NTHR * r) >> 3;
                st.xr[r] = (t0 + t < L) ? ld16(xc + xo[r]) : zero8();
            }
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                if (t0 + wtg * 8 + r < L) {
                    load_b_row(st.br[r], bc + r * (int)bstride);
                } else {
#pragma unroll
                    for (int k = 0; k < WD; ++k) st.br[r][k] = 0u;
                }
            }
        }
        const f32x4 *wp = reinterpret_cast<const f32x4 *>(wh + t0 + wtg * 8);
        st.w[0] = wp[0];
        st.w[1] = wp[1];
        st.glast = Gh[t0 + Q - 1];
    };
    auto commit = [&](const Stage &st) {
#pragma unroll
        for (int r = 0; r < XPC; ++r) {
            const int id = tid + NTHR * r;
            *reinterpret_cast<bf16x8 *>(&Xs[(id >> 3) * XP + (id & 7) * 8]) = st.xr[r];
        }
        // W: scale token row r by w_r, then pack the pair (2k, 2k+1) of column j
#pragma unroll
        for (int j = 0; j < WC; ++j) {
            u32x4 o;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t a = st.br[2 * k][j >> 1], bb = st.br[2 * k + 1][j >> 1];
                const float fa = (j & 1) ? bf_hi(a) : bf_lo(a);
                const float fb = (j & 1) ? bf_hi(bb) : bf_lo(bb);
                const float wa = st.w[k >> 1][2 * (k & 1)], wb = st.w[k >> 1][2 * (k & 1) + 1];
                o[k] = pack_bf16(fa * wa, fb * wb);
            }
            *reinterpret_cast<u32x4 *>(&WT[(wcg * WC + j) * PT + wtg * 8]) = o;
        }
        if (tid == 0) alph = fast_exp2(st.glast);
    };

    const int offW = (nh * 32 + (lane & 31)) * PT + 8 * (lane >> 5) + kh * (Q / KS);
    const int offX = tr_off_natural(lane, XP) + ph * 32 + kh * (Q / KS) * XP;
    float run = 1.0f;   // decay product since the group start (keeper thread)

    // One chunk: refill `refill` with chunk c+2, store the chunk-start state,
    // decay and accumulate chunk c from LDS, then (after everyone has read the
    // tile) write chunk c+1 from `next` into LDS and fold the K-halves.  Loads
    // and commits are unconditional (indices clamped to the group's last chunk;
    // the extra copies are never used) so the wait counts let the c+2 loads stay
    // in flight across the commit.
    auto step = [&](int c, const Stage &next, Stage &refill) {
        issue(refill, min(c + 2, c1 - 1));
        if (kh == 0) {
            bf16 *Sc = S + ((int64_t)bh * nc + c) * P * N + (int64_t)p_col * N + n_lane;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                bf16x4 o;
#pragma unroll
                for (int r = 0; r < 4; ++r) o[r] = (bf16)acc[4 * q + r];
                *reinterpret_cast<bf16x4 *>(Sc + 8 * q) = o;
            }
        }
        const float a = alph;
        if (keeper && beta != nullptr) {
            beta[(int64_t)bh * nc + c] = run;
            run *= a;
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[v] *= a;

        const bf16 *wt = WT + offW;
        const bf16 *xt = Xs + offX;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            const bf16x8 bf = cat8(tr_read4(xt + ks * 16 * XP), tr_read4(xt + (ks * 16 + 4) * XP));
            mma(acc, ld16(wt + ks * 16), bf);
        }
        __syncthreads();   // tile of chunk c consumed
        if constexpr (KS > 1) {
            if (kh == 1) {
#pragma unroll
                for (int v = 0; v < 16; ++v) red[((wave - 2 * NWN) * 16 + v) * 64 + lane] = acc[v];
            }
        }
        commit(next);
        __syncthreads();   // tile of chunk c+1 and the partial states visible
        if constexpr (KS > 1) {
            if (kh == 0) {
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[v] += red[(wave * 16 + v) * 64 + lane];
            } else {
                acc = zero_acc();
            }
        }
    };

    Stage sa, sb;
    issue(sa, c0);
    issue(sb, min(c0 + 1, c1 - 1));
    commit(sa);
    __syncthreads();
    int c = c0;
    for (; c + 1 < c1; c += 2) {
        step(c, sb, sa);
        step(c + 1, sa, sb);
    }
    if (c < c1) step(c, sb, sa);

    // acc (kh = 0 waves) now holds the state after the group's last chunk
    float *dst = (Ug != nullptr) ? Ug + ((int64_t)bh * ng + grp) * P * N : hT;
    if (dst != nullptr && (Ug != nullptr || hT != nullptr) && kh == 0) {
        const int64_t off = (Ug != nullptr) ? 0 : st_off;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            f32x4 o;
#pragma unroll
            for (int r = 0; r < 4; ++r) o[r] = acc[4 * q + r];
            *reinterpret_cast<f32x4 *>(dst + off + (int64_t)p_col * N + n_lane + 8 * q) = o;
        }
    }
    if (keeper && gam != nullptr) gam[(int64_t)bh * ng + grp] = run;
}

// ===========================================================================
// Group scan.  For each (batch*head, state element): walk the groups in order,
// H_1 = U_0 and H_{g+1} = gamma_g H_g + U_g; H_g (the true state at group g's
// start) replaces U_g in place, and the state after the last group is hT.
// ===========================================================================
__global__ __launch_bounds__(256) void group_scan_kernel(float *__restrict__ Ug,
                                                         const float *__restrict__ gam,
                                                         float *__restrict__ hT, int PN, int ng)
{
    const int bh = blockIdx.y;
    const int e = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (e >= PN) return;
    f32x4 hcar = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int g = 0; g < ng; ++g) {
        f32x4 *u = reinterpret_cast<f32x4 *>(Ug + ((int64_t)bh * ng + g) * PN + e);
        const f32x4 v = *u;
        if (g > 0) *u = hcar;
        const float gm = gam[(int64_t)bh * ng + g];
#pragma unroll
        for (int r = 0; r < 4; ++r) hcar[r] = gm * hcar[r] + v[r];
    }
    if (hT != nullptr) *reinterpret_cast<f32x4 *>(hT + (int64_t)bh * PN + e) = hcar;
}

// ===========================================================================
// Chunk output.  Workgroup = one (chunk, batch*head) with Q/32 waves; wave w
// owns one 32-token row tile I = rowtile(w).  Waves w and w + Q/64 (which the
// hardware places on the same SIMD) get tiles that add up to Q/32 - 1, so every
// SIMD does the same number, Q/32 + 1, of causal tile pairs (J, I), J <= I.
// Two waves per SIMD let one wave's loads, barriers and exponentials overlap
// the other's matrix products.  The output is built transposed, Y^T [64 p x 32
// tokens] per row tile.
//
// Phase 1 streams N in slices of 64: the slice of B (all chunk rows) and of S
// (all p) is staged in LDS, the wave's C rows come from global memory, and the
// next slice is loaded into registers while the current one is multiplied:
//   * CB_J = (B C^T)[tile J, tile I] for J <= I (accumulators indexed by J);
//   * Y^T += S C^T (the inter-chunk term).
// Phase 2, per J <= I: the C B^T tile becomes the decay matrix
//   M[j, i] = (i >= j) ? CB[j, i] * exp2(G_i - G_j) : 0      (selection, never a product with a mask)
// rounded to bf16 and fed to MFMA straight from registers against (dt x)^T.
// Off the diagonal (J < I) the decay factors exactly into
// exp2(G_i - G_e) * exp2(G_e - G_j), e the last token of tile J; both factors are
// <= 1, the second a per-token table, so such a tile costs one exp2 per lane.
// The Y^T accumulator is scaled by exp2(G_i) between the two phases.
//
// Chunk-start state handed over by a grouped state pass (Hg != NULL): S holds
// the state relative to the start of the chunk's group, to which beta_c H_g is
// added while staging (group 0 already started from the true initial state).
// ===========================================================================
template <int Q>
__global__ __launch_bounds__(2 * Q) void chunk_out_bf16_kernel(
    const bf16 *__restrict__ x, const bf16 *__restrict__ Bm, const bf16 *__restrict__ Cm,
    const float *__restrict__ G2, const float *__restrict__ dtT, const bf16 *__restrict__ S,
    const float *__restrict__ D, bf16 *__restrict__ y, const float *__restrict__ Hg,
    const float *__restrict__ beta, int L, int H, int G, int N, int nc, int Lp, int K, int ng,
    int xcd)
{
    constexpr int P = 64, NI = Q / 32, NW = Q / 32, NTHR = 2 * Q, NS = 64;
    constexpr int XP = Q + 8, BP = frag_pitch(NS), SP = frag_pitch(NS);
    constexpr int BPC = Q * (NS / 8) / NTHR;   // 16-byte B pieces per thread per slice
    constexpr int SPC = P * (NS / 8) / NTHR;   // 16-byte S pieces per thread per slice
    static_assert(BPC >= 1 && SPC >= 1, "slice staging cover");
    // (dt x)^T [p][position]: within each 16-token group the token at offset o is
    // kept at position o with its middle two 4-token blocks swapped, so the
    // accumulator token order 4(l/32)+{0..3}, 8+4(l/32)+{0..3} of lane l becomes 8
    // consecutive positions.
    __shared__ __attribute__((aligned(16))) bf16 Xd[P * XP];
    __shared__ __attribute__((aligned(16))) bf16 Bs[Q * BP];
    __shared__ __attribute__((aligned(16))) bf16 Ss[P * SP];
    __shared__ __attribute__((aligned(16))) float Gs[Q];
    __shared__ __attribute__((aligned(16))) float We[Q];   // exp2(G_e - G_j), e = end of j's tile

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int I = (w < NW / 2) ? w : NW - 1 - (w - NW / 2);

    // Workgroup -> (chunk, batch*head), heads innermost.  With `xcd` set (nc a
    // multiple of 8) XCD x gets the contiguous chunk range [x nc/8, (x+1) nc/8):
    // a chunk's B and C rows are shared by all its heads and a state-pass group's
    // carried state by its consecutive chunks, and both then stay in one L2.
    const int bH = gridDim.x / nc;
    int c, bh;
    if (xcd) {
        const int xx = blockIdx.x & 7, slot = blockIdx.x >> 3;
        c = xx * (nc / 8) + slot / bH;
        bh = slot % bH;
    } else {
        c = blockIdx.x / bH;
        bh = blockIdx.x % bH;
    }
    const int b = bh / H, h = bh % H, g = h / (H / G);
    const int t0 = c * Q;
    const bool full = t0 + Q <= L;
    const int64_t xstride = (int64_t)H * P, cstride = (int64_t)G * N;
    const bf16 *xb = x + ((int64_t)b * L + t0) * xstride + (int64_t)h * P;
    const bf16 *Bb = Bm + ((int64_t)b * L + t0) * cstride + (int64_t)g * N;
    const bf16 *Cb = Cm + ((int64_t)b * L + t0) * cstride + (int64_t)g * N;
    const bf16 *Sb = S + ((int64_t)bh * nc + c) * P * N;
    const float *Gh = G2 + (int64_t)bh * Lp + t0;
    const float *dh = dtT + (int64_t)bh * Lp + t0;
    const int kq = 8 * (lane >> 5);
    const int cgrp = (Hg != nullptr) ? c / K : 0;
    const float *Hc = (cgrp > 0) ? Hg + ((int64_t)bh * ng + cgrp) * P * N : nullptr;
    const float bc = (cgrp > 0) ? beta[(int64_t)bh * nc + c] : 0.0f;

    const int i_loc = I * 32 + (lane & 31);
    const bool iv = full || t0 + i_loc < L;
    const bf16 *crow = Cb + i_loc * (int)cstride + kq;

    // registers holding the next N slice while the current one is multiplied
    bf16x8 bq[BPC], sq[SPC], cn[NS / 16];
    f32x4 hq[SPC][2];
    auto load_slice = [&](int n0) {
        if (full) {   // uniform: no per-lane predication
#pragma unroll
            for (int r = 0; r < BPC; ++r) {
                const int id = tid + NTHR * r, t = id >> 3, oct = id & 7;
                bq[r] = ld16(Bb + t * (int)cstride + n0 + oct * 8);
            }
#pragma unroll
            for (int ks = 0; ks < NS / 16; ++ks) cn[ks] = ld16(crow + n0 + ks * 16);
        } else {
#pragma unroll
            for (int r = 0; r < BPC; ++r) {
                const int id = tid + NTHR * r, t = id >> 3, oct = id & 7;
                bq[r] = (t0 + t < L) ? ld16(Bb + t * (int)cstride + n0 + oct * 8) : zero8();
            }
#pragma unroll
            for (int ks = 0; ks < NS / 16; ++ks) cn[ks] = iv ? ld16(crow + n0 + ks * 16) : zero8();
        }
#pragma unroll
        for (int r = 0; r < SPC; ++r) {
            const int id = tid + NTHR * r, p = id >> 3, oct = id & 7;
            sq[r] = ld16(Sb + p * N + n0 + oct * 8);
            if (Hc != nullptr) {
                hq[r][0] = *reinterpret_cast<const f32x4 *>(Hc + p * N + n0 + oct * 8);
                hq[r][1] = *reinterpret_cast<const f32x4 *>(Hc + p * N + n0 + oct * 8 + 4);
            }
        }
    };

    // (dt x)^T tile and the chunk's decays; the first N slice is requested right
    // behind the x tile so both latencies overlap.  Thread = one 8-token x 4-p
    // block: rows loaded token-major, scaled by dt, packed per p column.  A wave
    // covers 8 token groups (lane % 8) x 8 column groups (lane / 8).
    {
        const int tg = (w >> 1) * 8 + (lane & 7), cg = (w & 1) * 8 + (lane >> 3);
        u32x2 xv[8];
        if (full) {
#pragma unroll
            for (int r = 0; r < 8; ++r)
                xv[r] = *reinterpret_cast<const u32x2 *>(xb + (tg * 8 + r) * (int)xstride + cg * 4);
        } else {
#pragma unroll
            for (int r = 0; r < 8; ++r)
                xv[r] = (t0 + tg * 8 + r < L)
                            ? *reinterpret_cast<const u32x2 *>(xb + (tg * 8 + r) * (int)xstride + cg * 4)
                            : u32x2{0u, 0u};
        }
        const f32x4 d0 = *reinterpret_cast<const f32x4 *>(dh + tg * 8);
        const f32x4 d1 = *reinterpret_cast<const f32x4 *>(dh + tg * 8 + 4);
        float gt = 0.0f, ge = 0.0f;
        if (tid < Q) {
            gt = Gh[tid];
            ge = Gh[tid | 31];
        }
        load_slice(0);
        const float d[8] = {d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
        // positions of this block's tokens: 8 tokens at offset 0 or 8 of a 16-group
        // -> two runs of 4 positions, 8 apart
        const int pos0 = (tg >> 1) * 16 + ((tg & 1) ? 4 : 0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            u32x2 lo, hi;
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const uint32_t a0 = xv[2 * k][j >> 1], a1 = xv[2 * k + 1][j >> 1];
                lo[k] = pack_bf16(((j & 1) ? bf_hi(a0) : bf_lo(a0)) * d[2 * k],
                                  ((j & 1) ? bf_hi(a1) : bf_lo(a1)) * d[2 * k + 1]);
                const uint32_t b0 = xv[4 + 2 * k][j >> 1], b1 = xv[5 + 2 * k][j >> 1];
                hi[k] = pack_bf16(((j & 1) ? bf_hi(b0) : bf_lo(b0)) * d[4 + 2 * k],
                                  ((j & 1) ? bf_hi(b1) : bf_lo(b1)) * d[5 + 2 * k]);
            }
            bf16 *row = Xd + (cg * 4 + j) * XP + pos0;
            *reinterpret_cast<u32x2 *>(row) = lo;
            *reinterpret_cast<u32x2 *>(row + 8) = hi;
        }
        if (tid < Q) {
            Gs[tid] = gt;
            We[tid] = fast_exp2(ge - gt);
        }
    }

    f32x16 cb[NI];
#pragma unroll
    for (int J = 0; J < NI; ++J) cb[J] = zero_acc();
    f32x16 ya[2] = {zero_acc(), zero_acc()};

    // ---------------- phase 1: C B^T tiles and S C^T over N slices ----------------
    for (int n0 = 0; n0 < N; n0 += NS) {
        __syncthreads();   // previous slice consumed; first time: Xd, Gs, We written
#pragma unroll
        for (int r = 0; r < BPC; ++r) {
            const int id = tid + NTHR * r, t = id >> 3, oct = id & 7;
            *reinterpret_cast<bf16x8 *>(&Bs[t * BP + oct * 8]) = bq[r];
        }
#pragma unroll
        for (int r = 0; r < SPC; ++r) {
            const int id = tid + NTHR * r, p = id >> 3, oct = id & 7;
            bf16x8 sv = sq[r];
            if (Hc != nullptr) {
#pragma unroll
                for (int e = 0; e < 8; ++e) sv[e] = (bf16)((float)sv[e] + bc * hq[r][e >> 2][e & 3]);
            }
            *reinterpret_cast<bf16x8 *>(&Ss[p * SP + oct * 8]) = sv;
        }
        bf16x8 cf[NS / 16];
#pragma unroll
        for (int ks = 0; ks < NS / 16; ++ks) cf[ks] = cn[ks];
        // next slice (the last iteration re-requests the last slice; never used)
        load_slice(min(n0 + NS, N - NS));
        __syncthreads();

#pragma unroll
        for (int J = 0; J < NI; ++J) {
            if (J <= I) {
                const bf16 *brow = Bs + (J * 32 + (lane & 31)) * BP + kq;
#pragma unroll
                for (int ks = 0; ks < NS / 16; ++ks)
                    mma(cb[J], *reinterpret_cast<const bf16x8 *>(brow + ks * 16), cf[ks]);
            }
        }
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
            const bf16 *srow = Ss + (pp * 32 + (lane & 31)) * SP + kq;
#pragma unroll
            for (int ks = 0; ks < NS / 16; ++ks)
                mma(ya[pp], *reinterpret_cast<const bf16x8 *>(srow + ks * 16), cf[ks]);
        }
    }

    // ---------------- phase 2: Y^T = exp2(G_i) Y^T + M (dt x) ----------------
    const float gi = Gs[i_loc];
    const float si = fast_exp2(gi);
#pragma unroll
    for (int v = 0; v < 16; ++v) { ya[0][v] *= si; ya[1][v] *= si; }
    const int offX = (lane & 31) * XP + 8 * (lane >> 5);
#pragma unroll
    for (int J = 0; J < NI; ++J) {
        if (J > I) continue;
        const int jrow = J * 32 + 4 * (lane >> 5);   // + 8q + r for element 4q + r
        bf16x8 m[2];
        if (J < I) {
            const float ci = fast_exp2(gi - Gs[J * 32 + 31]);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 we = *reinterpret_cast<const f32x4 *>(&We[jrow + 8 * q]);
#pragma unroll
                for (int r = 0; r < 4; ++r) m[q >> 1][4 * (q & 1) + r] = (bf16)(cb[J][4 * q + r] * we[r] * ci);
            }
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 gj = *reinterpret_cast<const f32x4 *>(&Gs[jrow + 8 * q]);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float val = cb[J][4 * q + r] * fast_exp2(gi - gj[r]);
                    m[q >> 1][4 * (q & 1) + r] = (bf16)((i_loc >= jrow + 8 * q + r) ? val : 0.0f);
                }
            }
        }
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            const bf16 *xt = Xd + offX + J * 32 + 16 * sub;
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) mma(ya[pp], ld16(xt + pp * 32 * XP), m[sub]);
        }
    }

    // ---------------- y = Y + D x ----------------
    if (iv) {
        const float Dh = D[h];
        const int yo = i_loc * (int)xstride;
        bf16 *yb = y + ((int64_t)b * L + t0) * xstride + (int64_t)h * P;
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int p = pp * 32 + 8 * q + 4 * (lane >> 5);
                const bf16x4 xv = *reinterpret_cast<const bf16x4 *>(xb + yo + p);
                bf16x4 o;
#pragma unroll
                for (int r = 0; r < 4; ++r) o[r] = (bf16)(ya[pp][4 * q + r] + Dh * (float)xv[r]);
                *reinterpret_cast<bf16x4 *>(yb + yo + p) = o;
            }
        }
    }
}

// ===========================================================================
// Launchers
// ===========================================================================
template <int Q>
static hipError_t sp_launch(const Shape &s, const void *x, const void *B, const float *G2,
                            const float *wT, const float *h0, void *S, float *hT, float *Ug,
                            float *gam, float *beta, int K, int ng, hipStream_t st)
{
    constexpr int NT = 32, KS = 2;
    const int ntiles = (int)(s.N / NT);
    const int bH = (int)(s.b * s.H);
    const int xcd = (bH % 8 == 0) ? 1 : 0;
    hipLaunchKernelGGL((state_pass_bf16_kernel<Q, NT, KS>), dim3((unsigned)(bH * ntiles * ng)),
                       dim3(64 * 2 * (NT / 32) * KS), 0, st, (const bf16 *)x, (const bf16 *)B, G2,
                       wT, h0, (bf16 *)S, hT, Ug, gam, beta, (int)s.L, (int)s.H, (int)s.G,
                       (int)s.N, (int)s.nc, (int)s.Lp, ntiles, K, ng, xcd);
    return hipGetLastError();
}

static hipError_t sp_dispatch(const Shape &s, const void *x, const void *B, const float *G2,
                              const float *wT, const float *h0, void *S, float *hT, float *Ug,
                              float *gam, float *beta, int K, int ng, hipStream_t st)
{
    switch (s.Q) {
    case 64: return sp_launch<64>(s, x, B, G2, wT, h0, S, hT, Ug, gam, beta, K, ng, st);
    case 128: return sp_launch<128>(s, x, B, G2, wT, h0, S, hT, Ug, gam, beta, K, ng, st);
    default: return sp_launch<256>(s, x, B, G2, wT, h0, S, hT, Ug, gam, beta, K, ng, st);
    }
}

hipError_t launch_state_pass_bf16(const Shape &s, const void *x, const void *B, const float *G2,
                                  const float *wT, const float *h0, void *S, float *hT,
                                  hipStream_t st)
{
    return sp_dispatch(s, x, B, G2, wT, h0, S, hT, nullptr, nullptr, nullptr, (int)s.nc, 1, st);
}

Grouping state_pass_groups(const Shape &s)
{
    Grouping gp;
    if (!s.bf16) {
        gp.K = (int)s.nc;
        gp.ng = 1;
        return gp;
    }
    // aim for about four state-pass workgroups per CU (two are resident at a
    // time) while keeping at least two chunks per group
    const int64_t units = s.b * s.H * (s.N / 32);
    int64_t ng = (1024 + units - 1) / units;
    ng = std::max<int64_t>(1, std::min<int64_t>(ng, s.nc / 2));
    const int64_t K = (s.nc + ng - 1) / ng;
    gp.K = (int)K;
    gp.ng = (int)((s.nc + K - 1) / K);
    return gp;
}

hipError_t launch_state_pass_grouped(const Shape &s, const Grouping &gp, const void *x,
                                     const void *B, const float *G2, const float *wT,
                                     const float *h0, void *S, float *hT, float *Ug, float *gam,
                                     float *beta, hipStream_t st)
{
    if (!s.bf16 || gp.ng <= 1) return launch_state_pass(s, x, B, G2, wT, h0, S, hT, st);
    hipError_t e = sp_dispatch(s, x, B, G2, wT, h0, S, nullptr, Ug, gam, beta, gp.K, gp.ng, st);
    if (e != hipSuccess) return e;
    const int PN = (int)(s.P * s.N);
    dim3 grid((unsigned)((PN / 4 + 255) / 256), (unsigned)(s.b * s.H));
    hipLaunchKernelGGL(group_scan_kernel, grid, dim3(256), 0, st, Ug, gam, hT, PN, gp.ng);
    return hipGetLastError();
}

template <int Q>
static hipError_t co_launch(const Shape &s, const void *x, const void *B, const void *C,
                            const float *G2, const float *dtT, const void *S, const float *D,
                            void *y, const float *Hg, const float *beta, int K, int ng,
                            hipStream_t st)
{
    const int xcd = (s.nc % 8 == 0) ? 1 : 0;
    hipLaunchKernelGGL((chunk_out_bf16_kernel<Q>), dim3((unsigned)(s.nc * s.b * s.H)), dim3(2 * Q), 0,
                       st, (const bf16 *)x, (const bf16 *)B, (const bf16 *)C, G2, dtT,
                       (const bf16 *)S, D, (bf16 *)y, Hg, beta, (int)s.L, (int)s.H, (int)s.G,
                       (int)s.N, (int)s.nc, (int)s.Lp, K, ng, xcd);
    return hipGetLastError();
}

hipError_t launch_chunk_out_bf16(const Shape &s, const void *x, const void *B, const void *C,
                                 const float *G2, const float *dtT, const void *S, const float *D,
                                 void *y, const float *Hg, const float *beta, int K, int ng,
                                 hipStream_t st)
{
    switch (s.Q) {
    case 64: return co_launch<64>(s, x, B, C, G2, dtT, S, D, y, Hg, beta, K, ng, st);
    case 128: return co_launch<128>(s, x, B, C, G2, dtT, S, D, y, Hg, beta, K, ng, st);
    default: return co_launch<256>(s, x, B, C, G2, dtT, S, D, y, Hg, beta, K, ng, st);
    }
}

}  // namespace ssd
