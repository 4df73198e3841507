// zc_table.cpp -- the library's exponent-code table generator (host C++).
//
// ZipCCL (arXiv 2604.27844), abstract, technique (1): the bf16 exponent is
// coded with a fixed code derived from the Gaussian law of training tensors,
// so no statistics are collected at run time.  The shd-paper.top summary
// (key-design paragraph) adds that frequent exponents get short code words.
//
// The code is for d = E_max - e, the distance of a value's exponent below the
// largest exponent of its 128-value group (a member of i.i.d. N(0, s^2)
// values).  With F(x) = P(|X| < x) and binade probabilities
// p_k = F(2^(k+1)) - F(2^k):
//   P(d = 0)   = sum_m p_m F(2^(m+1))^127
//   P(d = j)   = sum_m p_(m-j) [F(2^(m+1))^127 - F(2^m)^127]      (j >= 1)
//   P(d >= 16) = sum_m F(2^(m-15)) [F(2^(m+1))^127 - F(2^m)^127]
// averaged over 64 scale phases s = 2^((q + 1/2)/64) so that it holds for any
// scale.  Huffman lengths (equal weights: the earlier-created node is taken
// first) and canonical code values follow.
//
// This runs at build time (zc_table_emit writes the constants the kernels
// compile in) and again at run time for the self-check in zc_code_table().
#include "zc_table.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <queue>
#include <vector>

namespace zc {

namespace {

constexpr int kGroup = 128;
constexpr int kPhases = 64;

// Binade-max law at one scale, accumulated into w[0..16].
void accumulate_law(double sigma, double scale, double* w)
{
    const int lo = -90, hi = 50;
    std::vector<double> cdf(hi - lo + 2);
    for (int m = lo; m <= hi + 1; ++m)
        cdf[m - lo] = std::erf(std::ldexp(1.0, m) / (sigma * std::sqrt(2.0)));
    auto F = [&](int m) { return m < lo ? 0.0 : (m > hi + 1 ? 1.0 : cdf[m - lo]); };
    for (int m = lo + 20; m <= hi; ++m) {
        const double below = std::pow(F(m), kGroup - 1);
        const double upto = std::pow(F(m + 1), kGroup - 1);
        w[0] += scale * (F(m + 1) - F(m)) * upto;
        for (int j = 1; j < kEscapeFrom; ++j)
            w[j] += scale * (F(m - j + 1) - F(m - j)) * (upto - below);
        w[kEscape] += scale * F(m - kEscapeFrom + 1) * (upto - below);
    }
}

}  // namespace

void exponent_law(double* w)
{
    std::fill(w, w + kSymbols, 0.0);
    for (int q = 0; q < kPhases; ++q)
        accumulate_law(std::exp2((q + 0.5) / kPhases), 1.0 / kPhases, w);
}

void huffman(const double* w, int nsym, int* len)
{
    struct Node { double w; int id; };
    auto heavier = [](const Node& a, const Node& b) {
        return a.w != b.w ? a.w > b.w : a.id > b.id;
    };
    std::priority_queue<Node, std::vector<Node>, decltype(heavier)> pq(heavier);
    std::vector<int> up(2 * nsym, -1);
    for (int s = 0; s < nsym; ++s)
        pq.push({w[s], s});
    int next = nsym;
    while (pq.size() > 1) {
        Node a = pq.top(); pq.pop();
        Node b = pq.top(); pq.pop();
        up[a.id] = up[b.id] = next;
        pq.push({a.w + b.w, next++});
    }
    for (int s = 0; s < nsym; ++s) {
        int depth = 0;
        for (int x = s; up[x] >= 0; x = up[x])
            ++depth;
        len[s] = depth;
    }
}

void canonical(const int* len, int nsym, uint32_t* code)
{
    std::vector<int> order(nsym);
    for (int s = 0; s < nsym; ++s)
        order[s] = s;
    std::stable_sort(order.begin(), order.end(),
                     [&](int a, int b) { return len[a] < len[b]; });
    uint32_t c = 0;
    for (int r = 0; r < nsym; ++r) {
        const int s = order[r];
        if (r > 0)
            c = (c + 1) << (len[s] - len[order[r - 1]]);
        code[s] = c;
    }
}

bool build_table(Table* t)
{
    double w[kSymbols];
    exponent_law(w);
    huffman(w, kSymbols, t->len);
    canonical(t->len, kSymbols, t->code);
    for (int s = 0; s < kSymbols; ++s) {
        t->prob[s] = w[s];
        if (t->len[s] < 1 || t->len[s] > kMaxCodeLen)
            return false;
    }
    // Decoder lookup on the first kLutBits bits of the stream: symbol and
    // length of every code word no longer than kLutBits (both must fit a
    // nibble); 0 for prefixes of longer code words, which take the second
    // level.
    std::memset(t->lut, 0, sizeof t->lut);
    for (int s = 0; s < kSymbols; ++s) {
        const int L = t->len[s];
        if (L > kLutBits)
            continue;
        if (s > 15 || L > 15)
            return false;
        const uint32_t first = t->code[s] << (kLutBits - L);
        const uint32_t count = 1u << (kLutBits - L);
        for (uint32_t i = 0; i < count; ++i)
            t->lut[first + i] = static_cast<uint8_t>((s << 4) | L);
    }
    // Second level for the long code words (all must share the all-ones
    // prefix of kLutBits bits and fit in kLutBits + kTailBits bits).
    t->tail_ok = true;
    std::memset(t->tail, 0, sizeof t->tail);
    for (int s = 0; s < kSymbols; ++s) {
        const int L = t->len[s];
        if (L <= kLutBits)
            continue;
        if (L > kLutBits + kTailBits || (t->code[s] >> (L - kLutBits)) != (1u << kLutBits) - 1) {
            t->tail_ok = false;
            continue;
        }
        const int rest = L - kLutBits;                       // bits after the prefix
        const uint32_t low = t->code[s] & ((1u << rest) - 1);
        const uint32_t first = low << (kTailBits - rest);
        for (uint32_t i = 0; i < (1u << (kTailBits - rest)); ++i)
            t->tail[first + i] = static_cast<uint16_t>((s << 8) | L);
    }
    for (int i = 0; i < (1 << kTailBits); ++i)
        if (t->tail[i] == 0)
            t->tail_ok = false;
    // Per-length canonical ranges for the long code words: a window whose
    // first L bits are v (left-aligned in 32 bits) holds a code word of
    // length L if v < limit[L]; its symbol is sym[v - base[L]].
    std::vector<int> order(kSymbols);
    for (int s = 0; s < kSymbols; ++s)
        order[s] = s;
    std::stable_sort(order.begin(), order.end(),
                     [&](int a, int b) { return t->len[a] < t->len[b]; });
    for (int r = 0; r < kSymbols; ++r)
        t->sorted_sym[r] = static_cast<uint8_t>(order[r]);
    int r = 0;
    for (int L = 0; L <= kMaxCodeLen; ++L) {
        t->limit[L] = 0;
        t->base[L] = 0;
    }
    for (int L = 1; L <= kMaxCodeLen; ++L) {
        int first_rank = r;
        while (r < kSymbols && t->len[order[r]] == L)
            ++r;
        if (r == first_rank) {
            // no code word of this length: nothing below it can match here
            t->limit[L] = (L == 1) ? 0u
                         : (t->limit[L - 1] << 1);
            t->base[L] = 0;
            continue;
        }
        const uint32_t first_code = t->code[order[first_rank]];
        t->limit[L] = first_code + static_cast<uint32_t>(r - first_rank);
        // symbol rank = v - first_code + first_rank
        t->base[L] = static_cast<int32_t>(first_code) - first_rank;
    }
    return true;
}

}  // namespace zc
