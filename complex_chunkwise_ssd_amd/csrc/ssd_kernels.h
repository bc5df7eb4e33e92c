// ssd_kernels.h -- gfx950 kernels of the complex chunkwise SSD scan.
//
// The method (Mamba-3-Lite pages, "Extending" guide Path A Step 1 and Path B
// Step 2, index.html lab 03): per (batch row b, head h)
//   a_t      = softplus(dt_t) * A_h
//   s_t      = exp(a_t) s_{t-1} + B_t x_t^T,     y_t = Re(C_t^T s_t)
// evaluated chunk by chunk. Inside a chunk of Q tokens with running sums
// Lam[l] = a_0 + ... + a_l (relative to the chunk start):
//   Y_diag[l] = sum_{s<=l} (C_l . B_s) exp(Lam[l] - Lam[s]) x_s     (intra-chunk)
//   Y_off[l]  = exp(Lam[l]) C_l^T H_c                               (state-to-output)
//   H_{c+1}   = exp(Lam[Q-1]) H_c + sum_s exp(Lam[Q-1] - Lam[s]) B_s x_s^T
//
// scan_kernel runs one workgroup (eight wave64s) per (b, h, segment, 64-wide
// slice of D) and walks its chunks in order, so the N x 64 state H never
// leaves registers. Every contraction is a real-split fp32 MFMA 16x16x4:
//   G^T = B C^T (complex, K = N)      tile rows s, columns l
//   M   = G o L                       elementwise on the accumulator
//   Y  += Re(M X) + Re(C' H)          M and H feed the next MFMA straight from
//                                     their accumulator layout
//   H   = decay H + B^T (decay' X)    K = chunk rows
// The exponents of L are formed from running sums restarted on each 16-row
// tile, so no difference of two long running sums is ever taken.
#pragma once

#include <ssd_device.h>
#include <ssd_plan.h>

namespace ssd {

SSD_DEVICE float softplus_f(float v) { return fmaxf(v, 0.f) + log1pf(expf(-fabsf(v))); }

SSD_DEVICE v2f cmul(v2f a, v2f b) { return v2f{a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x}; }

SSD_DEVICE v2f cexp_f(v2f z)
{
    float s, c;
    sincosf(z.y, &s, &c);
    const float m = expf(z.x);
    return v2f{m * c, m * s};
}

// ------------------------------------------------------------ discretisation

// A_bar[i] = exp(softplus(dt[i]) * A[i % H]) over the flattened (batch, T, H).
SSD_KERNEL(256) void discretise_abar_kernel(const float *dt, const float *A, int64_t n, int H,
                                            float *abar)
{
    const int64_t i = block_id() * 256 + thread_id();
    if (i >= n)
        return;
    const int h = (int)(i % H);
    const float sp = softplus_f(dt[i]);
    const v2f a = v2f{A[2 * h] * sp, A[2 * h + 1] * sp};
    *(v2f *)&abar[2 * i] = cexp_f(a);
}

// Lambda[b, h, c, l] = sum_{j<=l} softplus(dt[b, cQ+j, h]) * A[h]; one thread
// per (b, c, h), h fastest so that the dt reads of a wave are contiguous.
SSD_KERNEL(256) void discretise_cumsum_kernel(const float *dt, const float *A, int B, int T, int H,
                                              int Q, int nc, float *lam)
{
    const int64_t i = block_id() * 256 + thread_id();
    if (i >= (int64_t)B * nc * H)
        return;
    const int h = (int)(i % H);
    const int c = (int)((i / H) % nc);
    const int b = (int)(i / ((int64_t)H * nc));
    const v2f Ah = v2f{A[2 * h], A[2 * h + 1]};
    v2f run = v2f{0.f, 0.f};
    float *out = lam + (((int64_t)b * H + h) * nc + c) * (int64_t)Q * 2;
    for (int l = 0; l < Q; ++l) {
        const int t = c * Q + l;
        if (t < T) {
            const float sp = softplus_f(dt[((int64_t)b * T + t) * H + h]);
            run.x += sp * Ah.x;
            run.y += sp * Ah.y;
        }
        *(v2f *)&out[2 * l] = run;
    }
}

// final_state = initial_state (or zero) for T == 0.
SSD_KERNEL(256) void copy_state_kernel(const float *src, float *dst, int64_t n)
{
    const int64_t i = block_id() * 256 + thread_id();
    if (i < n)
        dst[i] = src ? src[i] : 0.f;
}

// ------------------------------------------------------------------ the scan

// Chunk tile pair of causal tile k (0 <= k < NR(NR+1)/2): the NR diagonal tiles
// first, then the strictly lower ones (st < lt) by increasing lt.
SSD_DEVICE void tile_pair(int k, int nr, int &st, int &lt)
{
    if (k < nr) {
        st = lt = k;
        return;
    }
    int idx = k - nr;
    lt = 1;
    while (idx >= lt) {
        idx -= lt;
        ++lt;
    }
    st = idx;
}

// R: chunk rows held on chip (chunk_size rounded up to 16, 32 or 64; extra
// rows are identity padding). FULL: produce y and the final state; otherwise
// only the zero-start end state and total log-decay of each segment.
template <int R, bool FULL>
SSD_KERNEL(kThreads) void scan_kernel(ScanParams p)
{
    constexpr int NR = R / 16;               // 16-row tiles per chunk
    constexpr int NT = NR * (NR + 1) / 2;    // causal tile pairs
    constexpr int LDB = kNPad + 4;           // [row][n] plane stride (floats)
    constexpr int LDT = R + 4;               // [n][row] plane stride (floats)
    constexpr int LOADS = R * (kNPad / 2) / kThreads;  // 16-byte loads per thread per B or C tile
    static_assert(LOADS >= 1, "tile too small for the thread count");

    SSD_LDS float sBre[FULL ? R * LDB : 1], sBim[FULL ? R * LDB : 1];  // B[s][n]
    SSD_LDS float sCre[FULL ? R * LDB : 1], sCim[FULL ? R * LDB : 1];  // C[l][n]
    SSD_LDS float sTre[kNPad * LDT], sTim[kNPad * LDT];                // B[s][n] stored at [n][s]
    SSD_LDS v4f sMre[FULL ? NT * 64 : 1], sMim[FULL ? NT * 64 : 1];    // M tiles, lane-major
    SSD_LDS v4f sYx[FULL ? 4 * NR * 64 : 1];                           // partial-y exchange
    SSD_LDS v2f sLam[R];       // running sum of a inside the 16-row tile (inclusive)
    SSD_LDS v2f sEin[R];       // exp(Lam[l]) from the chunk start
    SSD_LDS v2f sDout[R];      // exp(sum of a over rows s+1 .. end of chunk)
    SSD_LDS v2f sV[R];         // exp(sum of a over rows s+1 .. end of its tile)
    SSD_LDS v2f sU[R * NR];    // exp(sum of a over rows after tile st .. l), st < tile(l)
    SSD_LDS v2f sDecay[1];     // exp(sum of a over the chunk)

    const int tid = thread_id();
    const int lane = tid & 63;
    const int w = wave_id();
    const int dtl = w & 3;     // 16-column tile of the D slice
    const int nh = w >> 2;     // half of the state rows (32 of 64)
    const int Lr = lane & 15;
    const int Lk = lane >> 4;

    int64_t blk = block_id();
    const int db = (int)(blk % p.ndb);
    blk /= p.ndb;
    const int seg = (int)(blk % p.groups_per_seq);
    blk /= p.groups_per_seq;
    const int h = (int)(blk % p.H);
    const int b = (int)(blk / p.H);

    const int64_t row0 = (int64_t)b * p.T * p.H + h;  // flat (b, t=0, h) index
    const int64_t sx = (int64_t)p.H * p.D;            // token stride of x and y
    const int64_t sbc = (int64_t)p.H * p.N;           // token stride of B_t and C_t
    const float *xb = p.x + (row0 * p.D + (int64_t)db * kDBlock) * 2;
    const float *Bb = p.Bt + row0 * p.N * 2;
    const float *Cb = p.Ct + row0 * p.N * 2;
    const float *dtb = p.dt + row0;
    const v2f Ah = v2f{p.A[2 * h], p.A[2 * h + 1]};
    const int dcol = db * kDBlock + 16 * dtl + Lr;    // this lane's column of D
    const bool dvalid = dcol < p.D;
    const int64_t bh = (int64_t)b * p.H + h;

    // State rows n = 16 * (2 * nh + i) + 4 * Lk + r, column dcol.
    v4f Hre[2], Him[2];
    for (int i = 0; i < 2; ++i) {
        Hre[i] = v4f{0.f, 0.f, 0.f, 0.f};
        Him[i] = v4f{0.f, 0.f, 0.f, 0.f};
    }
    auto add_state = [&](const float *base, v2f scale) {
        // H = scale * H + base[n, dcol] over this lane's elements (base may be null).
        for (int i = 0; i < 2; ++i)
            for (int r = 0; r < 4; ++r) {
                const int n = 16 * (2 * nh + i) + 4 * Lk + r;
                v2f e = v2f{0.f, 0.f};
                if (base && n < p.N && dvalid)
                    e = *(const v2f *)&base[((int64_t)n * p.D + dcol) * 2];
                const v2f hv = cmul(scale, v2f{Hre[i][r], Him[i][r]});
                Hre[i][r] = hv.x + e.x;
                Him[i][r] = hv.y + e.y;
            }
    };
    if (FULL) {
        if (p.init_state)
            add_state(p.init_state + bh * p.N * p.D * 2, v2f{0.f, 0.f});
        for (int q = 0; q < seg; ++q) {
            const int64_t sidx = bh * (p.P - 1) + q;
            const v2f lg = *(const v2f *)&p.seg_logdecay[sidx * 2];
            add_state(p.seg_state + sidx * p.N * p.D * 2, cexp_f(lg));
        }
    }

    const int c_begin = seg * p.spc;
    const int c_end = c_begin + p.spc < p.nc ? c_begin + p.spc : p.nc;
    v2f seg_log = v2f{0.f, 0.f};

    // Registers holding the next chunk's inputs while the current one runs.
    v4f pB[LOADS], pC[LOADS];
    float pdt = 0.f;
    v2f pX[NR][4];
    auto fetch = [&](int c) {
        const int t0 = c * p.Q;
        const int rows = p.Q < p.T - t0 ? p.Q : p.T - t0;
        for (int i = 0; i < LOADS; ++i) {
            const int e = i * kThreads + tid;
            const int row = e >> 5;
            const int n = (e & 31) * 2;
            const bool ok = row < rows && n < p.N;
            const int64_t off = ((int64_t)(t0 + row) * sbc + n) * 2;
            pB[i] = ok ? *(const v4f *)&Bb[off] : v4f{0.f, 0.f, 0.f, 0.f};
            if (FULL)
                pC[i] = ok ? *(const v4f *)&Cb[off] : v4f{0.f, 0.f, 0.f, 0.f};
        }
        if (w == 0)
            pdt = lane < rows ? dtb[(int64_t)(t0 + lane) * p.H] : 0.f;
        for (int q = 0; q < NR; ++q)
            for (int j = 0; j < 4; ++j) {
                const int s = 16 * q + 4 * Lk + j;
                const bool ok = s < rows && dvalid;
                pX[q][j] = ok ? *(const v2f *)&xb[((int64_t)(t0 + s) * sx + 16 * dtl + Lr) * 2]
                              : v2f{0.f, 0.f};
            }
    };

    if (c_begin < c_end)
        fetch(c_begin);

    for (int c = c_begin; c < c_end; ++c) {
        const int t0 = c * p.Q;
        const int rows = p.Q < p.T - t0 ? p.Q : p.T - t0;

        // ---- stage 1 (wave 0): per-token log-decay and the decay factors.
        if (w == 0) {
            const float sp = softplus_f(pdt);
            const v2f a = lane < rows ? v2f{Ah.x * sp, Ah.y * sp} : v2f{0.f, 0.f};
            v2f lam = a;  // inclusive running sum inside the 16-row tile
            v2f rs = a;   // inclusive running sum towards the end of the tile
            for (int off = 1; off < 16; off <<= 1) {
                const float ux = shfl_up16(lam.x, off), uy = shfl_up16(lam.y, off);
                const float dx = shfl_down16(rs.x, off), dy = shfl_down16(rs.y, off);
                if (Lr >= off) {
                    lam.x += ux;
                    lam.y += uy;
                }
                if (Lr + off < 16) {
                    rs.x += dx;
                    rs.y += dy;
                }
            }
            const float sgx = shfl_down16(rs.x, 1), sgy = shfl_down16(rs.y, 1);
            const v2f sig = Lr < 15 ? v2f{sgx, sgy} : v2f{0.f, 0.f};  // rows s+1 .. tile end
            v2f tau[NR];
            for (int t = 0; t < NR; ++t)
                tau[t] = v2f{shfl_idx(lam.x, 16 * t + 15), shfl_idx(lam.y, 16 * t + 15)};
            v2f pre = v2f{0.f, 0.f}, post = v2f{0.f, 0.f}, tot = v2f{0.f, 0.f};
            for (int t = 0; t < NR; ++t) {
                tot += tau[t];
                if (t < Lk)
                    pre += tau[t];
                if (t > Lk)
                    post += tau[t];
            }
            if (lane < R) {
                sLam[lane] = lam;
                sEin[lane] = cexp_f(lam + pre);
                sDout[lane] = cexp_f(sig + post);
                sV[lane] = cexp_f(sig);
                for (int st = 0; st < NR; ++st) {
                    if (st < Lk) {
                        v2f z = lam;
                        for (int t = st + 1; t < Lk; ++t)
                            z += tau[t];
                        sU[lane * NR + st] = cexp_f(z);
                    }
                }
            }
            if (lane == 0)
                sDecay[0] = cexp_f(tot);
            seg_log += tot;
        }

        // ---- stage 2 (all): chunk inputs into LDS planes, x into registers.
        for (int i = 0; i < LOADS; ++i) {
            const int e = i * kThreads + tid;
            const int row = e >> 5;
            const int n = (e & 31) * 2;
            const v4f vb = pB[i];
            if (FULL) {
                const v4f vc = pC[i];
                *(v2f *)&sBre[row * LDB + n] = v2f{vb.x, vb.z};
                *(v2f *)&sBim[row * LDB + n] = v2f{vb.y, vb.w};
                *(v2f *)&sCre[row * LDB + n] = v2f{vc.x, vc.z};
                *(v2f *)&sCim[row * LDB + n] = v2f{vc.y, vc.w};
            }
            sTre[n * LDT + row] = vb.x;
            sTim[n * LDT + row] = vb.y;
            sTre[(n + 1) * LDT + row] = vb.z;
            sTim[(n + 1) * LDT + row] = vb.w;
        }
        v2f X[NR][4];
        for (int q = 0; q < NR; ++q)
            for (int j = 0; j < 4; ++j)
                X[q][j] = pX[q][j];
        block_sync();
        if (c + 1 < c_end)
            fetch(c + 1);

        v4f Y[NR];
        if (FULL) {
            // ---- phase 1a: M tiles = (B C^T)^T o L^T, produced round-robin by the waves.
            for (int k = w; k < NT; k += 8) {
                int st, lt;
                tile_pair(k, NR, st, lt);
                v4f gre = v4f{0.f, 0.f, 0.f, 0.f}, gim = v4f{0.f, 0.f, 0.f, 0.f};
                for (int q = 0; q < kNPad / 16; ++q) {
                    const int col = 16 * q + 4 * Lk;
                    const v4f bre = *(const v4f *)&sBre[(16 * st + Lr) * LDB + col];
                    const v4f bim = *(const v4f *)&sBim[(16 * st + Lr) * LDB + col];
                    const v4f cre = *(const v4f *)&sCre[(16 * lt + Lr) * LDB + col];
                    const v4f cim = *(const v4f *)&sCim[(16 * lt + Lr) * LDB + col];
                    for (int j = 0; j < 4; ++j) {
                        gre = mfma_16x16x4(bre[j], cre[j], gre);
                        gre = mfma_16x16x4(bim[j], -cim[j], gre);
                        gim = mfma_16x16x4(bre[j], cim[j], gim);
                        gim = mfma_16x16x4(bim[j], cre[j], gim);
                    }
                }
                // Accumulator element r of this lane: s = 16 st + 4 Lk + r, l = 16 lt + Lr.
                const int l = 16 * lt + Lr;
                v4f mre, mim;
                for (int r = 0; r < 4; ++r) {
                    const int s = 16 * st + 4 * Lk + r;
                    v2f L;
                    if (st == lt) {
                        const bool causal = Lr >= 4 * Lk + r;
                        const v2f dl = causal ? sLam[l] - sLam[s] : v2f{0.f, 0.f};
                        L = cexp_f(dl);
                        if (!causal)
                            L = v2f{0.f, 0.f};
                    } else {
                        L = cmul(sU[l * NR + st], sV[s]);
                    }
                    const v2f m = cmul(v2f{gre[r], gim[r]}, L);
                    mre[r] = m.x;
                    mim[r] = m.y;
                }
                sMre[k * 64 + lane] = mre;
                sMim[k * 64 + lane] = mim;
            }

            // ---- phase 1b: state-to-output term Re(C' H) with C' = exp(Lam) C, this
            // wave's half of the state rows.
            for (int lt = 0; lt < NR; ++lt) {
                Y[lt] = v4f{0.f, 0.f, 0.f, 0.f};
                const v2f e = sEin[16 * lt + Lr];
                for (int i = 0; i < 2; ++i) {
                    const int col = 16 * (2 * nh + i) + 4 * Lk;
                    const v4f cre = *(const v4f *)&sCre[(16 * lt + Lr) * LDB + col];
                    const v4f cim = *(const v4f *)&sCim[(16 * lt + Lr) * LDB + col];
                    for (int r = 0; r < 4; ++r) {
                        const float ar = cre[r] * e.x - cim[r] * e.y;
                        const float ain = -(cre[r] * e.y + cim[r] * e.x);
                        Y[lt] = mfma_16x16x4(ar, Hre[i][r], Y[lt]);
                        Y[lt] = mfma_16x16x4(ain, Him[i][r], Y[lt]);
                    }
                }
            }
        }

        // ---- phase 1c: H = exp(sum a) H + B^T (decay' o X).
        {
            const v2f g = sDecay[0];
            for (int i = 0; i < 2; ++i)
                for (int r = 0; r < 4; ++r) {
                    const v2f hv = cmul(g, v2f{Hre[i][r], Him[i][r]});
                    Hre[i][r] = hv.x;
                    Him[i][r] = hv.y;
                }
            for (int q = 0; q < NR; ++q) {
                v2f xs[4];
                for (int j = 0; j < 4; ++j)
                    xs[j] = cmul(sDout[16 * q + 4 * Lk + j], X[q][j]);
                for (int i = 0; i < 2; ++i) {
                    const int n = 16 * (2 * nh + i) + Lr;
                    const v4f tre = *(const v4f *)&sTre[n * LDT + 16 * q + 4 * Lk];
                    const v4f tim = *(const v4f *)&sTim[n * LDT + 16 * q + 4 * Lk];
                    for (int j = 0; j < 4; ++j) {
                        Hre[i] = mfma_16x16x4(tre[j], xs[j].x, Hre[i]);
                        Hre[i] = mfma_16x16x4(tim[j], -xs[j].y, Hre[i]);
                        Him[i] = mfma_16x16x4(tre[j], xs[j].y, Him[i]);
                        Him[i] = mfma_16x16x4(tim[j], xs[j].x, Him[i]);
                    }
                }
            }
        }
        block_sync();

        if (FULL) {
            // ---- phase 2: intra-chunk term Re(M X); tiles split between the two
            // waves that share this column tile.
            for (int k = nh; k < NT; k += 2) {
                int st, lt;
                tile_pair(k, NR, st, lt);
                const v4f mre = sMre[k * 64 + lane];
                const v4f mim = sMim[k * 64 + lane];
                for (int r = 0; r < 4; ++r) {
                    Y[lt] = mfma_16x16x4(mre[r], X[st][r].x, Y[lt]);
                    Y[lt] = mfma_16x16x4(mim[r], -X[st][r].y, Y[lt]);
                }
            }
            // Row tile lt is finished and stored by the wave with nh == lt % 2.
            for (int lt = 0; lt < NR; ++lt)
                if ((lt & 1) != nh)
                    sYx[(dtl * NR + lt) * 64 + lane] = Y[lt];
            block_sync();
            for (int lt = 0; lt < NR; ++lt) {
                if ((lt & 1) != nh)
                    continue;
                const v4f o = sYx[(dtl * NR + lt) * 64 + lane];
                for (int r = 0; r < 4; ++r) {
                    const int l = 16 * lt + 4 * Lk + r;
                    if (l < rows && dvalid)
                        p.y[(row0 + (int64_t)(t0 + l) * p.H) * p.D + dcol] = Y[lt][r] + o[r];
                }
            }
        }
    }

    // ---- results of the segment.
    float *out = nullptr;
    if (FULL) {
        if (seg == p.P - 1 && p.final_state)
            out = p.final_state + bh * p.N * p.D * 2;
    } else {
        const int64_t sidx = bh * (p.P - 1) + seg;
        out = p.seg_state + sidx * p.N * p.D * 2;
        if (db == 0 && tid == 0)
            *(v2f *)&p.seg_logdecay[sidx * 2] = seg_log;
    }
    if (out) {
        for (int i = 0; i < 2; ++i)
            for (int r = 0; r < 4; ++r) {
                const int n = 16 * (2 * nh + i) + 4 * Lk + r;
                if (n < p.N && dvalid)
                    *(v2f *)&out[((int64_t)n * p.D + dcol) * 2] = v2f{Hre[i][r], Him[i][r]};
            }
    }
}

}  // namespace ssd
