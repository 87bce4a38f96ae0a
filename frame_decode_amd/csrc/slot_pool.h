// Host side of the fixed-shape session slots (PersonaPlex 7B page, "A
// server built around the conversation clock": all sessions advance on one
// clock in fixed-shape batches; new sessions fill free slots without
// changing what the GPU runs).  Pure host code.
//
// Every operation validates all of its arguments before changing anything,
// so a failed call leaves the pool as it was.
#pragma once

#include <algorithm>
#include <cstdint>
#include <numeric>
#include <vector>

#include "../../include/fd.h"

namespace fd {

// Largest frame index a rolling-window session may reach (2^30 frames of
// 80 ms: about 2.7 years).
constexpr int kRollingMaxFrame = 1 << 30;

class SlotPool {
public:
    // rolling: sessions continue past max_context frames (the cache keeps the
    // last max_context); otherwise a full window stops the step.
    SlotPool(int n_slots, int max_context, bool rolling = false)
        : active_(n_slots, 0), pos_(n_slots, 0), stale_(n_slots, 0), max_context_(max_context),
          rolling_(rolling) {}

    int size() const { return (int)active_.size(); }
    int max_context() const { return max_context_; }

    // n lowest-numbered free slots, ascending; all or nothing.
    fd_status alloc(int n, int32_t* out) {
        if (n < 0 || (n > 0 && !out)) return FD_E_INVAL;
        std::vector<int32_t> pick;
        for (int s = 0; s < size() && (int)pick.size() < n; ++s)
            if (!active_[s]) pick.push_back(s);
        if ((int)pick.size() < n) return FD_E_NOSLOT;
        for (int i = 0; i < n; ++i) {
            active_[pick[i]] = 1;
            pos_[pick[i]] = 0;
            stale_[pick[i]] = 0;
            out[i] = pick[i];
        }
        dirty_ = dirty_ || n > 0;
        return FD_OK;
    }

    // Marks the listed slots free; rejects out-of-range, unallocated and
    // repeated ids without changing anything.
    fd_status free(const int32_t* ids, int n) {
        if (n < 0 || (n > 0 && !ids)) return FD_E_INVAL;
        std::vector<char> seen(size(), 0);
        for (int i = 0; i < n; ++i) {
            int s = ids[i];
            if (s < 0 || s >= size() || !active_[s] || seen[s]) return FD_E_BADSLOT;
            seen[s] = 1;
        }
        for (int i = 0; i < n; ++i) {
            active_[ids[i]] = 0;
            stale_[ids[i]] = 0;
        }
        dirty_ = dirty_ || n > 0;
        return FD_OK;
    }

    fd_status set_position(int s, int p) {
        if (s < 0 || s >= size() || !active_[s]) return FD_E_BADSLOT;
        if (p < 0 || p > (rolling_ ? kRollingMaxFrame : max_context_)) return FD_E_INVAL;
        pos_[s] = p;
        stale_[s] = 0;
        dirty_ = true;
        return FD_OK;
    }

    // A step that stopped early (a persistent-walk barrier timed out) left
    // the device positions and the new cache entries of every active slot
    // unknown: those slots stay stale until the caller gives each a
    // position (set_position) or frees it.
    void mark_stale() {
        for (int s = 0; s < size(); ++s)
            if (active_[s]) stale_[s] = 1;
    }

    bool any_stale(int* which) const {
        for (int s = 0; s < size(); ++s)
            if (active_[s] && stale_[s]) {
                if (which) *which = s;
                return true;
            }
        return false;
    }

    fd_status state(int s, int32_t* a, int32_t* p) const {
        if (s < 0 || s >= size()) return FD_E_BADSLOT;
        if (a) *a = active_[s];
        if (p) *p = pos_[s];
        return FD_OK;
    }

    // True if some active slot's window is full (the step may not run); a
    // rolling window is full only at the largest frame index.
    bool any_full(int* which) const {
        const int cap = rolling_ ? kRollingMaxFrame : max_context_;
        for (int s = 0; s < size(); ++s)
            if (active_[s] && pos_[s] >= cap) {
                if (which) *which = s;
                return true;
            }
        return false;
    }

    // After a step: every active slot's position advances by one (the
    // device does the same on its copy).
    void advance() {
        for (int s = 0; s < size(); ++s)
            if (active_[s]) ++pos_[s];
    }

    int n_active() const {
        int n = 0;
        for (int a : active_) n += a;
        return n;
    }

    bool dirty() const { return dirty_; }
    void clear_dirty() { dirty_ = false; }
    void mark_dirty() { dirty_ = true; }

    // Device image: int32 active[S], int32 pos[S], then int32 order[S]: the
    // active slots by descending position (ties by slot), then the inactive
    // ones ascending.  Attention takes its (slot, head) tasks in this order,
    // so the longest windows start first and the shortest fill the last
    // round (positions advance together between uploads, so the order
    // holds until the next change).
    void image(int32_t* dst) const {
        const int n = size();
        for (int s = 0; s < n; ++s) {
            dst[s] = active_[s];
            dst[n + s] = pos_[s];
        }
        int32_t* order = dst + 2 * n;
        std::iota(order, order + n, 0);
        std::stable_sort(order, order + n, [&](int32_t a, int32_t b) {
            if (active_[a] != active_[b]) return active_[a] > active_[b];
            return active_[a] && pos_[a] > pos_[b];
        });
    }

private:
    std::vector<int32_t> active_;
    std::vector<int32_t> pos_;
    std::vector<char> stale_;
    int max_context_;
    bool rolling_;
    bool dirty_ = true;
};

}  // namespace fd
