"""CPU oracle of the KDA decode update.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the CPU
baseline leg of the benchmark are its only users.  The product library never
imports, links or calls anything here, and nothing here imports the product.
"""
