// pack.cpp — the example packer ("No Padding Please", §V, §V-A, §IX-B (packing algorithm details, Algorithm 1))
// and the padded-stack baseline (§VII-C), as integer host code.
//
// Shelf packing: examples are bucketed by height and the buckets visited from
// the tallest; a row takes, each time, the widest example of the current
// bucket that still fits after a separator (equal widths: lowest index); only
// when nothing of the current bucket fits is the row closed, so a row may run
// on into the next, shorter bucket. Rows are then stacked with
// separator rows in between, examples top-aligned, and the row still open at
// the end is kept. Canvas width = max(canvas_w_min, widest example).
// The exact-height mode (§V: one height per packed row, which the input-skewing
// trick of §IV-A needs) also closes the row when its bucket is used up.
#include <algorithm>
#include <cstring>
#include <numeric>

#include "layout.h"
#include "../../include/mdlstm.h"

namespace mdl {

namespace {

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

void paint_maps(Layout& L) {
    const int64_t P = (int64_t)L.Hc * L.Wc;
    L.eid.assign(P, -1);
    L.border.assign(P, 0);
    for (int e = 0; e < L.n; ++e) {
        const int32_t* r = &L.rect[4 * e];
        for (int y = r[0]; y < r[0] + r[2]; ++y)
            for (int x = r[1]; x < r[1] + r[3]; ++x) L.eid[(int64_t)y * L.Wc + x] = e;
    }
    for (int y = 0; y < L.Hc; ++y)
        for (int x = 0; x < L.Wc; ++x) {
            const int64_t p = (int64_t)y * L.Wc + x;
            const int e = L.eid[p];
            if (e < 0) continue;
            uint8_t bits = 0;
            if (x > 0 && L.eid[p - 1] == e) bits |= 1;
            if (x + 1 < L.Wc && L.eid[p + 1] == e) bits |= 2;
            if (y > 0 && L.eid[p - L.Wc] == e) bits |= 4;
            if (y + 1 < L.Hc && L.eid[p + L.Wc] == e) bits |= 8;
            L.border[p] = bits;
        }
}

// Cuts the computed cells of all examples (example order, row-major inside each region) into G ranges of
// nearly equal size (G as the constants in layout.h set it), with boundaries on multiples of 32 cells of
// the sequence; each range's pieces inside one example are its segments. A range that would hold more than kGroupSegs
// segments is closed early and its rest goes on in a new group. Depends only on the layout, so the
// weight-gradient sums are blocked the same way on every run.
void split_wgrad(Layout& L) {
    L.segs.clear();
    L.groups.assign(1, 0);
    const int64_t T = L.computed_cells;
    int64_t G = std::max<int64_t>(1, std::min<int64_t>(kGroups, (T + kGroupMinCells - 1) / kGroupMinCells));
    if (G >= kGroupRound) G = G / kGroupRound * kGroupRound;
    int e = 0;
    int64_t pos = 0;
    for (int64_t g = 0; g < G; ++g) {
        const int64_t end = g + 1 == G ? T : std::min(T, (T * (g + 1) / G + 31) / 32 * 32);
        int in_group = 0;
        while (pos < end) {
            while (L.cell_off[e + 1] <= pos) ++e;
            const int64_t stop = std::min(end, L.cell_off[e + 1]);
            if (in_group == kGroupSegs) {
                L.groups.push_back((int32_t)(L.segs.size() / 3));
                in_group = 0;
            }
            L.segs.push_back(e);
            L.segs.push_back((int32_t)(pos - L.cell_off[e]));
            L.segs.push_back((int32_t)(stop - L.cell_off[e]));
            ++in_group;
            pos = stop;
        }
        if (in_group > 0) L.groups.push_back((int32_t)(L.segs.size() / 3));
    }
    L.nsegs = (int32_t)(L.segs.size() / 3);
    L.ngroups = (int32_t)L.groups.size() - 1;
    std::vector<int32_t> key(L.ngroups, 0);
    for (int g = 0; g < L.ngroups; ++g)
        for (int sg = L.groups[g]; sg < L.groups[g + 1]; ++sg) {
            const int32_t* r = &L.rect[4 * L.segs[3 * sg]];
            key[g] = std::max(key[g], r[2] + r[3] - 1);
        }
    L.gorder.resize(4 * (size_t)L.ngroups);
    std::iota(L.gorder.begin(), L.gorder.end(), 0);
    std::stable_sort(L.gorder.begin(), L.gorder.end(),
                     [&](int32_t a, int32_t b) { return key[a >> 2] < key[b >> 2]; });
}

// The direction sum's chunks in readiness order (Layout::dsum).
void split_dsum(Layout& L) {
    std::vector<int32_t> ord(L.n);
    std::iota(ord.begin(), ord.end(), 0);
    auto depth = [&](int32_t e) { return L.rect[4 * e + 2] + L.rect[4 * e + 3] - 1; };
    std::stable_sort(ord.begin(), ord.end(), [&](int32_t a, int32_t b) { return depth(a) < depth(b); });
    L.dsum.clear();
    for (const int32_t e : ord) {
        const int64_t np = (int64_t)L.real[4 * e + 2] * L.real[4 * e + 3];
        for (int64_t p0 = 0; p0 < np; p0 += kSumChunk) {
            L.dsum.push_back(e);
            L.dsum.push_back((int32_t)p0);
            L.dsum.push_back((int32_t)std::min<int64_t>(np, p0 + kSumChunk));
        }
    }
    L.nsum = (int32_t)(L.dsum.size() / 3);
}

void finish(Layout& L) {
    const int n = L.n;
    L.flat_off.assign(n + 1, 0);
    L.cell_off.assign(n + 1, 0);
    L.max_depth = 0;
    L.max_diag = 0;
    for (int e = 0; e < n; ++e) {
        const int32_t* r = &L.rect[4 * e];
        const int32_t* q = &L.real[4 * e];
        L.flat_off[e + 1] = L.flat_off[e] + (int64_t)q[2] * q[3];
        L.cell_off[e + 1] = L.cell_off[e] + (int64_t)r[2] * r[3];
        L.max_depth = std::max(L.max_depth, r[2] + r[3] - 1);
        L.max_diag = std::max(L.max_diag, std::min(r[2], r[3]));
    }
    L.real_pixels = L.flat_off[n];
    L.computed_cells = L.cell_off[n];
    // unit schedule: (example, direction) pairs, most cells first (largest-first
    // list scheduling of independent chains), ties by example then direction
    L.units.resize(4 * n);
    std::iota(L.units.begin(), L.units.end(), 0);
    std::stable_sort(L.units.begin(), L.units.end(), [&](int32_t a, int32_t b) {
        const int64_t ca = (int64_t)L.rect[4 * (a >> 2) + 2] * L.rect[4 * (a >> 2) + 3];
        const int64_t cb = (int64_t)L.rect[4 * (b >> 2) + 2] * L.rect[4 * (b >> 2) + 3];
        return ca > cb;
    });
    paint_maps(L);
    split_wgrad(L);
    split_dsum(L);

    DescOffsets& o = L.off;
    size_t p = 0;
    o.rect = p;     p = align256(p + sizeof(int32_t) * 4 * n);
    o.real = p;     p = align256(p + sizeof(int32_t) * 4 * n);
    o.flat_off = p; p = align256(p + sizeof(int64_t) * (n + 1));
    o.cell_off = p; p = align256(p + sizeof(int64_t) * (n + 1));
    o.units = p;    p = align256(p + sizeof(int32_t) * 4 * n);
    o.segs = p;     p = align256(p + sizeof(int32_t) * L.segs.size());
    o.groups = p;   p = align256(p + sizeof(int32_t) * L.groups.size());
    o.gorder = p;   p = align256(p + sizeof(int32_t) * L.gorder.size());
    o.dsum = p;     p = align256(p + sizeof(int32_t) * L.dsum.size());
    o.eid = p;      p = align256(p + sizeof(int32_t) * (size_t)L.Hc * L.Wc);
    o.border = p;   p = align256(p + (size_t)L.Hc * L.Wc);
    o.total = p;
    L.host_desc.assign(o.eid, 0);
    std::memcpy(&L.host_desc[o.rect], L.rect.data(), sizeof(int32_t) * 4 * n);
    std::memcpy(&L.host_desc[o.real], L.real.data(), sizeof(int32_t) * 4 * n);
    std::memcpy(&L.host_desc[o.flat_off], L.flat_off.data(), sizeof(int64_t) * (n + 1));
    std::memcpy(&L.host_desc[o.cell_off], L.cell_off.data(), sizeof(int64_t) * (n + 1));
    std::memcpy(&L.host_desc[o.units], L.units.data(), sizeof(int32_t) * 4 * n);
    std::memcpy(&L.host_desc[o.segs], L.segs.data(), sizeof(int32_t) * L.segs.size());
    std::memcpy(&L.host_desc[o.groups], L.groups.data(), sizeof(int32_t) * L.groups.size());
    std::memcpy(&L.host_desc[o.gorder], L.gorder.data(), sizeof(int32_t) * L.gorder.size());
    std::memcpy(&L.host_desc[o.dsum], L.dsum.data(), sizeof(int32_t) * L.dsum.size());
}

}  // namespace

int build_layout(const int32_t* heights, const int32_t* widths, int32_t n, int32_t canvas_w_min,
                 int32_t sep, int32_t mode, Layout& L, std::string& err) {
    if (!heights || !widths) { err = "mdl_pack: null size array"; return MDL_EINVAL; }
    if (n < 1) { err = "mdl_pack: need n >= 1 examples"; return MDL_EINVAL; }
    if (mode != MDL_PACK_ALG1 && mode != MDL_PACK_PADDED && mode != MDL_PACK_EXACT) {
        err = "mdl_pack: unknown mode";
        return MDL_EINVAL;
    }
    if (sep < 0 || canvas_w_min < 1) { err = "mdl_pack: need sep >= 0 and canvas_w_min >= 1"; return MDL_EINVAL; }
    int32_t hmax = 0, wmax = 0;
    for (int e = 0; e < n; ++e) {
        if (heights[e] < 1 || widths[e] < 1) { err = "mdl_pack: example sizes must be >= 1"; return MDL_EINVAL; }
        hmax = std::max(hmax, heights[e]);
        wmax = std::max(wmax, widths[e]);
    }
    L = Layout();
    L.n = n;
    L.mode = mode;
    L.sep = sep;
    L.canvas_w_min = canvas_w_min;
    L.rect.assign(4 * (size_t)n, 0);
    L.real.assign(4 * (size_t)n, 0);

    if (mode == MDL_PACK_PADDED) {
        const int64_t Hc = (int64_t)n * hmax;
        if (Hc * wmax >= (int64_t(1) << 31)) { err = "mdl_pack: padded canvas exceeds 2^31 pixels"; return MDL_EOVERFLOW; }
        L.Hc = (int32_t)Hc;
        L.Wc = wmax;
        for (int e = 0; e < n; ++e) {
            int32_t* r = &L.rect[4 * e];
            int32_t* q = &L.real[4 * e];
            r[0] = q[0] = e * hmax;
            r[1] = q[1] = 0;
            r[2] = hmax; r[3] = wmax;
            q[2] = heights[e]; q[3] = widths[e];
            L.rows.push_back({e});
        }
        finish(L);
        return MDL_OK;
    }

    const int32_t Wc = std::max(canvas_w_min, wmax);
    // Step 1 of §V-A: buckets of equal height, filled tallest first. Step 2: rows take the widest example of
    // the bucket that still fits. With each bucket ordered widest first (equal widths in input order), that
    // example is the first one in this order that fits, and since a row only grows, whatever a scan passes
    // over cannot fit later in the same row: one scan over what is left of the bucket fills the current row,
    // and the row closes if the scan leaves anything. A scan that takes the whole bucket leaves the row open
    // for the next, shorter bucket.
    std::vector<int32_t> order(n);
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
        return heights[a] != heights[b] ? heights[a] > heights[b] : widths[a] > widths[b];
    });
    std::vector<int32_t> x0(n, 0), row, queue, rest;
    int64_t x_end = 0;
    for (int i = 0; i < n;) {
        int j = i;
        while (j < n && heights[order[j]] == heights[order[i]]) ++j;
        queue.assign(order.begin() + i, order.begin() + j);
        while (!queue.empty()) {
            rest.clear();
            for (int32_t e : queue) {
                const int64_t off = row.empty() ? 0 : x_end + sep;
                if (off + widths[e] <= Wc) {
                    x0[e] = (int32_t)off;
                    row.push_back(e);
                    x_end = off + widths[e];
                } else {
                    rest.push_back(e);
                }
            }
            queue.swap(rest);
            if (!queue.empty()) {  // nothing left in the bucket fits: the row is full
                L.rows.push_back(row);
                row.clear();
                x_end = 0;
            }
        }
        if (mode == MDL_PACK_EXACT && !row.empty()) {  // exact-height rows end with their bucket
            L.rows.push_back(row);
            row.clear();
            x_end = 0;
        }
        i = j;
    }
    if (!row.empty()) L.rows.push_back(row);

    int64_t y = 0, Hc = 0;
    std::vector<int64_t> y0(n, 0);
    for (const auto& r : L.rows) {
        for (int32_t e : r) y0[e] = y;
        Hc = y + heights[r[0]];
        y = Hc + sep;
    }
    if (Hc * Wc >= (int64_t(1) << 31)) { err = "mdl_pack: canvas exceeds 2^31 pixels"; return MDL_EOVERFLOW; }
    L.Hc = (int32_t)Hc;
    L.Wc = Wc;
    for (int e = 0; e < n; ++e) {
        int32_t* r = &L.rect[4 * e];
        r[0] = (int32_t)y0[e];
        r[1] = x0[e];
        r[2] = heights[e];
        r[3] = widths[e];
        std::memcpy(&L.real[4 * e], r, 4 * sizeof(int32_t));
    }
    finish(L);
    return MDL_OK;
}

}  // namespace mdl
