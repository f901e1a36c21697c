// pagepool.cpp -- host-side page allocator of a paged KV pool with
// copy-on-write (ForkKV Guide, "The Copy-on-Write Paradigm": forked sequences
// share pages read-only; the first write to a shared page goes to a freshly
// allocated private copy; "Reference Counting and Eviction": each page counts
// the sequences that hold it and returns to the pool when none does).
//
// The pool object only does the bookkeeping: reference counts, a free list and
// the page-level plan of an append.  It never touches device memory; the data
// movement of an append (the private copy and the new rows) is
// rattn_append_kv's kernel.  All entry points validate their arguments before
// changing anything, and a failed call leaves the pool and the table as they
// were.  One mutex per pool serialises calls from several threads.
#include <stdint.h>

#include <mutex>
#include <new>
#include <vector>

#include "rattn.h"

struct rattn_pagepool {
    int64_t n_pages;
    std::vector<int32_t> ref;   // sequences holding each page (0: free)
    std::vector<int32_t> free;  // free pages, taken from the back
    std::mutex mu;
};

namespace {

bool valid_page(const rattn_pagepool *p, int64_t page) { return page >= 0 && page < p->n_pages; }

}  // namespace

extern "C" {

int rattn_pagepool_create(int64_t n_pages, rattn_pagepool **out) {
    if (!out) return RATTN_E_NULL;
    if (n_pages < 1 || n_pages > INT32_MAX) return RATTN_E_SHAPE;
    rattn_pagepool *p = new (std::nothrow) rattn_pagepool;
    if (!p) return RATTN_E_POOL;
    try {
        p->n_pages = n_pages;
        p->ref.assign((size_t)n_pages, 0);
        p->free.resize((size_t)n_pages);
        // lowest page numbers first
        for (int64_t i = 0; i < n_pages; ++i) p->free[(size_t)i] = (int32_t)(n_pages - 1 - i);
    } catch (...) {
        delete p;
        return RATTN_E_POOL;
    }
    *out = p;
    return RATTN_OK;
}

void rattn_pagepool_destroy(rattn_pagepool *p) { delete p; }

int64_t rattn_pagepool_free_pages(rattn_pagepool *p) {
    if (!p) return RATTN_E_NULL;
    std::lock_guard<std::mutex> g(p->mu);
    return (int64_t)p->free.size();
}

int rattn_pagepool_refcount(rattn_pagepool *p, int32_t page, int32_t *count) {
    if (!p || !count) return RATTN_E_NULL;
    std::lock_guard<std::mutex> g(p->mu);
    if (!valid_page(p, page)) return RATTN_E_SHAPE;
    *count = p->ref[(size_t)page];
    return RATTN_OK;
}

int rattn_pagepool_alloc(rattn_pagepool *p, int64_t n, int32_t *pages) {
    if (!p || (n > 0 && !pages)) return RATTN_E_NULL;
    if (n < 0) return RATTN_E_SHAPE;
    std::lock_guard<std::mutex> g(p->mu);
    if ((int64_t)p->free.size() < n) return RATTN_E_POOL;
    for (int64_t i = 0; i < n; ++i) {
        const int32_t pg = p->free.back();
        p->free.pop_back();
        p->ref[(size_t)pg] = 1;
        pages[i] = pg;
    }
    return RATTN_OK;
}

int rattn_pagepool_retain(rattn_pagepool *p, const int32_t *pages, int64_t n) {
    if (!p || (n > 0 && !pages)) return RATTN_E_NULL;
    if (n < 0) return RATTN_E_SHAPE;
    std::lock_guard<std::mutex> g(p->mu);
    // a page listed k times gains k references
    for (int64_t i = 0; i < n; ++i)
        if (!valid_page(p, pages[i]) || p->ref[(size_t)pages[i]] < 1 || p->ref[(size_t)pages[i]] > INT32_MAX - n)
            return RATTN_E_SHAPE;
    for (int64_t i = 0; i < n; ++i) ++p->ref[(size_t)pages[i]];
    return RATTN_OK;
}

int rattn_pagepool_release(rattn_pagepool *p, const int32_t *pages, int64_t n) {
    if (!p || (n > 0 && !pages)) return RATTN_E_NULL;
    if (n < 0) return RATTN_E_SHAPE;
    std::lock_guard<std::mutex> g(p->mu);
    // every listing needs a reference to drop (a page listed k times needs k)
    std::vector<int32_t> drop;
    try {
        drop.assign((size_t)p->n_pages, 0);
    } catch (...) {
        return RATTN_E_POOL;
    }
    for (int64_t i = 0; i < n; ++i) {
        if (!valid_page(p, pages[i])) return RATTN_E_SHAPE;
        if (++drop[(size_t)pages[i]] > p->ref[(size_t)pages[i]]) return RATTN_E_SHAPE;
    }
    for (int64_t i = 0; i < n; ++i) {
        const int32_t pg = pages[i];
        if (--p->ref[(size_t)pg] == 0) p->free.push_back(pg);
    }
    return RATTN_OK;
}

int rattn_pagepool_plan_append(rattn_pagepool *p, int32_t *table, int64_t table_cap, int64_t cur_len,
                               int64_t n_new, int32_t page_size, int32_t *cow_src, int32_t *cow_dst) {
    if (!p || !table || !cow_src || !cow_dst) return RATTN_E_NULL;
    if (page_size < 1 || cur_len < 0 || n_new < 0 || table_cap < 0) return RATTN_E_SHAPE;
    const int64_t old_pages = (cur_len + page_size - 1) / page_size;
    const int64_t new_pages = (cur_len + n_new + page_size - 1) / page_size;
    if (new_pages > table_cap) return RATTN_E_SHAPE;
    std::lock_guard<std::mutex> g(p->mu);
    for (int64_t i = 0; i < old_pages; ++i)
        if (!valid_page(p, table[i]) || p->ref[(size_t)table[i]] < 1) return RATTN_E_SHAPE;
    *cow_src = -1;
    *cow_dst = -1;
    if (n_new == 0) return RATTN_OK;
    // the partly filled last page is written: in place when this sequence holds
    // it alone, else into a private copy
    const bool partial = cur_len % page_size != 0;
    const bool copy = partial && p->ref[(size_t)table[old_pages - 1]] > 1;
    const int64_t need = (new_pages - old_pages) + (copy ? 1 : 0);
    if ((int64_t)p->free.size() < need) return RATTN_E_POOL;
    if (copy) {
        const int32_t src = table[old_pages - 1];
        const int32_t dst = p->free.back();
        p->free.pop_back();
        p->ref[(size_t)dst] = 1;
        --p->ref[(size_t)src];  // still >= 1: another sequence holds it
        table[old_pages - 1] = dst;
        *cow_src = src;
        *cow_dst = dst;
    }
    for (int64_t i = old_pages; i < new_pages; ++i) {
        const int32_t pg = p->free.back();
        p->free.pop_back();
        p->ref[(size_t)pg] = 1;
        table[i] = pg;
    }
    return RATTN_OK;
}

}  // extern "C"
