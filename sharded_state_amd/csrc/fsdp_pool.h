// fsdp_pool.h -- the host worker pool of libfsdp_shard.so, shared by the
// offloaded optimizer step (fsdp_offload.cpp) and the shard-file reader
// (fsdp_ckpt.cpp).  Not installed.
#pragma once

#include <algorithm>
#include <condition_variable>
#include <cstdint>
#include <functional>
#include <mutex>
#include <thread>
#include <vector>

namespace fsdp {

// A fixed set of host threads that runs one job at a time: fn(w) for worker
// w = 0 .. k-1, worker 0 being the calling thread.
class Pool {
public:
    static Pool& get() {
        static Pool pool;
        return pool;
    }
    void run_workers(int k, const std::function<void(int)>& fn) {
        if (k <= 1) {
            fn(0);
            return;
        }
        std::lock_guard<std::mutex> serial(run_mu_);   // one job at a time
        while ((int)threads_.size() < k - 1) threads_.emplace_back([this] { loop(); });
        {
            std::lock_guard<std::mutex> lk(mu_);
            job_ = &fn;
            next_ = 1;
            workers_ = k;
            pending_ = k - 1;
            ++gen_;
        }
        cv_.notify_all();
        fn(0);
        std::unique_lock<std::mutex> lk(mu_);
        done_cv_.wait(lk, [&] { return pending_ == 0; });
        job_ = nullptr;
    }
    // fn(lo, hi) over [0, n) in `parts` contiguous ranges of whole 64-element groups.
    void run(int64_t n, int parts, const std::function<void(int64_t, int64_t)>& fn) {
        if (parts <= 1 || n < 2 * 4096) {
            fn(0, n);
            return;
        }
        const int64_t per = ((n + parts - 1) / parts + 63) / 64 * 64;
        const int k = (int)((n + per - 1) / per);
        run_workers(k, [&](int w) { fn(w * per, std::min(n, (w + 1) * per)); });
    }

private:
    void loop() {
        uint64_t seen = 0;
        std::unique_lock<std::mutex> lk(mu_);
        for (;;) {
            cv_.wait(lk, [&] { return stop_ || (gen_ != seen && next_ < workers_); });
            if (stop_) return;
            const int w = next_++;
            if (next_ >= workers_) seen = gen_;
            const std::function<void(int)>* job = job_;
            lk.unlock();
            (*job)(w);
            lk.lock();
            if (--pending_ == 0) done_cv_.notify_one();
        }
    }
    ~Pool() {
        {
            std::lock_guard<std::mutex> lk(mu_);
            stop_ = true;
        }
        cv_.notify_all();
        for (auto& t : threads_) t.join();
    }
    std::mutex run_mu_, mu_;
    std::condition_variable cv_, done_cv_;
    std::vector<std::thread> threads_;
    const std::function<void(int)>* job_ = nullptr;
    int next_ = 0, workers_ = 0, pending_ = 0;
    uint64_t gen_ = 0;
    bool stop_ = false;
};

}  // namespace fsdp
