// Host-side paged cache allocator: fixed-size pages handed to sequences on demand, reference
// counts with copy-on-write for shared prefixes, free space kept as coalesced extents that are
// split on allocation, and an emergency reserve for allocations that must not fail.
//
// Pages cited: "How the Ascend Computing Platform Achieves Same-Day Inference Adaptation for
// Ultra-Large Sparse Models" (SameDay) §3.1 (fixed-size blocks indexed directly by the sparse
// selection; reference counting and copy-on-write for requests sharing a prefix), §3.2 (blocks
// acquired incrementally during decoding and reclaimed as soon as no request references them),
// §4.3 (coalescing and splitting of free blocks; an emergency pool for severe fragmentation).
#include <algorithm>
#include <map>
#include <mutex>
#include <vector>

#include "../../include/sa.h"

struct sa_pool {
    int32_t num_pages = 0, page_size = 0, reserve = 0;
    int32_t free_pages = 0;
    std::map<int32_t, int32_t> extents;  // free runs: first page -> length (never adjacent)
    std::vector<int32_t> refcnt;         // per page: sequences holding it
    struct Seq {
        bool alive = false;
        int32_t len = 0;
        std::vector<int32_t> pages;
    };
    std::vector<Seq> seqs;
    std::mutex mu;

    // return one page to the free runs, merging with the runs that touch it
    void release_page(int32_t p) {
        auto next = extents.lower_bound(p);
        int32_t start = p, len = 1;
        if (next != extents.begin()) {
            auto prev = std::prev(next);
            if (prev->first + prev->second == p) {
                start = prev->first;
                len += prev->second;
                extents.erase(prev);
            }
        }
        if (next != extents.end() && next->first == p + 1) {
            len += next->second;
            extents.erase(next);
        }
        extents[start] = len;
        ++free_pages;
    }

    // take page p out of the run that holds it, splitting the run
    void take_page(int32_t p) {
        auto it = std::prev(extents.upper_bound(p));
        const int32_t start = it->first, len = it->second;
        extents.erase(it);
        if (p > start) extents[start] = p - start;
        if (p + 1 < start + len) extents[p + 1] = start + len - (p + 1);
        refcnt[p] = 1;
        --free_pages;
    }

    bool page_free(int32_t p) const {
        auto it = extents.upper_bound(p);
        if (it == extents.begin()) return false;
        --it;
        return p < it->first + it->second;
    }

    // n pages for a sequence whose last page is `after` (-1 if none): the page right after it
    // when free (the sequence stays contiguous), then the smallest run that holds the rest
    // (best fit), then the largest runs; the last `reserve` free pages only for urgent requests
    bool allocate(int32_t n, int32_t after, bool urgent, std::vector<int32_t> &out) {
        if (n <= 0) return true;
        if (free_pages - n < (urgent ? 0 : reserve)) return false;
        while (n > 0) {
            int32_t p = -1;
            if (after >= 0 && after + 1 < num_pages && page_free(after + 1)) {
                p = after + 1;
            } else {
                auto best = extents.end();
                for (auto it = extents.begin(); it != extents.end(); ++it)
                    if (it->second >= n && (best == extents.end() || it->second < best->second)) best = it;
                if (best == extents.end())  // no run holds all: start on the largest
                    best = std::max_element(extents.begin(), extents.end(),
                                            [](const auto &a, const auto &b) { return a.second < b.second; });
                p = best->first;
            }
            take_page(p);
            out.push_back(p);
            after = p;
            --n;
        }
        return true;
    }

    bool valid(int32_t s) const { return s >= 0 && s < (int32_t)seqs.size() && seqs[s].alive; }

    int32_t new_seq() {
        for (size_t i = 0; i < seqs.size(); ++i)
            if (!seqs[i].alive) {
                seqs[i] = Seq{true, 0, {}};
                return (int32_t)i;
            }
        seqs.push_back(Seq{true, 0, {}});
        return (int32_t)seqs.size() - 1;
    }
};

extern "C" {

sa_pool *sa_pool_create(int32_t num_pages, int32_t page_size, int32_t emergency_pages) {
    if (num_pages < 1 || page_size < 1 || emergency_pages < 0 || emergency_pages > num_pages) return nullptr;
    sa_pool *p = new sa_pool();
    p->num_pages = num_pages;
    p->page_size = page_size;
    p->reserve = emergency_pages;
    p->refcnt.assign(num_pages, 0);
    p->extents[0] = num_pages;
    p->free_pages = num_pages;
    return p;
}

void sa_pool_destroy(sa_pool *p) { delete p; }

sa_status sa_pool_stats(sa_pool *p, int32_t *free_pages, int32_t *free_runs, int32_t *largest_run) {
    if (!p) return SA_ERR_INVALID;
    std::lock_guard<std::mutex> g(p->mu);
    int32_t largest = 0;
    for (const auto &e : p->extents) largest = std::max(largest, e.second);
    if (free_pages) *free_pages = p->free_pages;
    if (free_runs) *free_runs = (int32_t)p->extents.size();
    if (largest_run) *largest_run = largest;
    return SA_OK;
}

int32_t sa_seq_new(sa_pool *p) {
    if (!p) return -1;
    std::lock_guard<std::mutex> g(p->mu);
    return p->new_seq();
}

int32_t sa_seq_fork(sa_pool *p, int32_t parent) {
    if (!p) return -1;
    std::lock_guard<std::mutex> g(p->mu);
    if (!p->valid(parent)) return -1;
    const int32_t c = p->new_seq();
    p->seqs[c].len = p->seqs[parent].len;
    p->seqs[c].pages = p->seqs[parent].pages;
    for (int32_t pg : p->seqs[c].pages) ++p->refcnt[pg];
    return c;
}

sa_status sa_seq_reserve(sa_pool *p, int32_t seq, int32_t new_len, int32_t urgent,
                         int32_t *copies, int32_t max_copies, int32_t *n_copies) {
    if (!p || !n_copies) return SA_ERR_INVALID;
    std::lock_guard<std::mutex> g(p->mu);
    *n_copies = 0;
    if (!p->valid(seq) || new_len < 0) return SA_ERR_INVALID;
    auto &s = p->seqs[seq];
    if (new_len <= s.len) return SA_OK;
    const int32_t P = p->page_size;
    const int32_t need = (new_len + P - 1) / P - (int32_t)s.pages.size();
    // the page that receives the first new token is shared: copy on write
    const bool cow = s.len % P != 0 && p->refcnt[s.pages.back()] > 1;
    if (cow && max_copies < 1) return SA_ERR_INVALID;
    std::vector<int32_t> got;
    const int32_t last = s.pages.empty() ? -1 : s.pages.back();
    if (!p->allocate(need + (cow ? 1 : 0), last, urgent != 0, got)) return SA_ERR_WORKSPACE;
    size_t k = 0;
    if (cow) {
        const int32_t old = s.pages.back(), fresh = got[k++];
        --p->refcnt[old];
        s.pages.back() = fresh;
        copies[0] = old;
        copies[1] = fresh;
        *n_copies = 1;
    }
    for (; k < got.size(); ++k) s.pages.push_back(got[k]);
    s.len = new_len;
    return SA_OK;
}

sa_status sa_seq_free(sa_pool *p, int32_t seq) {
    if (!p) return SA_ERR_INVALID;
    std::lock_guard<std::mutex> g(p->mu);
    if (!p->valid(seq)) return SA_ERR_INVALID;
    for (int32_t pg : p->seqs[seq].pages)
        if (--p->refcnt[pg] == 0) p->release_page(pg);
    p->seqs[seq] = sa_pool::Seq{};
    return SA_OK;
}

int32_t sa_seq_len(sa_pool *p, int32_t seq) {
    if (!p) return -1;
    std::lock_guard<std::mutex> g(p->mu);
    return p->valid(seq) ? p->seqs[seq].len : -1;
}

sa_status sa_seq_page_table(sa_pool *p, int32_t seq, int32_t *out, int32_t max_pages,
                            int32_t *n_pages) {
    if (!p || !out || !n_pages) return SA_ERR_INVALID;
    std::lock_guard<std::mutex> g(p->mu);
    if (!p->valid(seq)) return SA_ERR_INVALID;
    const auto &pg = p->seqs[seq].pages;
    *n_pages = (int32_t)pg.size();
    if ((int32_t)pg.size() > max_pages) return SA_ERR_WORKSPACE;
    std::copy(pg.begin(), pg.end(), out);
    return SA_OK;
}

int32_t sa_pool_refcount(sa_pool *p, int32_t page) {
    if (!p) return -1;
    std::lock_guard<std::mutex> g(p->mu);
    return page >= 0 && page < p->num_pages ? p->refcnt[page] : -1;
}

}  // extern "C"
