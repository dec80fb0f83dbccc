set -o pipefail
mkdir -p gpurun_out
timeout -k 10 600 python -u -m pytest tests/test_gpu_tiny.py tests/test_gpu_bf16.py -x -q --timeout 300 --timeout-method thread > gpurun_out/t3.log 2>&1 || { tail -30 gpurun_out/t3.log; exit 1; }
tail -2 gpurun_out/t3.log
timeout -k 10 400 python -u bench.py --steps 20 --warmup 4 --no-cpu-baseline > gpurun_out/b3.log 2>&1 || { tail -20 gpurun_out/b3.log; exit 1; }
tail -1 gpurun_out/b3.log | python -c "import json,sys; d=json.loads(sys.stdin.read()); r=d.pop('roofline'); d.pop('config'); d.pop('metric'); print(d); print(r)"
timeout -k 10 120 _work/probe2 > gpurun_out/probe2.log 2>&1 || { tail -5 gpurun_out/probe2.log; exit 1; }
cat gpurun_out/probe2.log
